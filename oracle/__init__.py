"""Plain CPU oracle for one GPT-2 training micro-step and optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or helpers with the HIP implementation and imports nothing from it.

The oracle is slow on purpose: materialised T x T attention per head, dense
logits per row chunk, a hand-written backward that follows the chain rule
step by step, and the optimizer written out element-wise.  It is generic over
the NumPy float dtype (float32 for parity runs, float64 for the finite
difference pins).

Sources (cited by page title and section throughout):
  [train-124M]   "How I trained my own GPT-2 124M on FineWeb-Edu" (vedasamhith.tech)
  [zero2front]   "GPT" chapter of Zero to Frontier (zerotofrontier.app/gpt)
  [repro-124M]   "Reproduce GPT-2 124M 复盘" (zhoudianfu.github.io)
  [fast-1gpu]    "Build an LLM From Scratch: Making Training Fast on One GPU" (vidyal.ai)
  [grad-accum]   "Multi-GPU calculation of gradients for accelerated training" (joelfernandes.org)

``oracle.modern`` holds the modern variant of the same model (RMSNorm,
rotary position embedding, SwiGLU, no position table, no biases) that
[repro-124M] trains; it reuses this package's attention and cross-entropy.

Every function in this package is pinned by a ``-m "not gpu"`` test against
something other than itself (finite differences, closed forms, invariants,
the worked examples the pages print, published known-answer vectors).
"""

from .model import (  # noqa: F401
    Config,
    param_specs,
    n_params,
    is_decayed,
    gelu_tanh,
    gelu_tanh_grad,
    layernorm_fwd,
    layernorm_bwd,
    packed_mask,
    packed_rows,
    attention_fwd,
    attention_bwd,
    cross_entropy_fwd_bwd,
    forward,
    fwd_bwd,
    lmhead_ce,
    lmhead_ce_sampled,
)
from .optim import global_grad_norm, clip_coef, adamw_update, clip_adamw_step  # noqa: F401
from .init import philox4x32_10, normal_from_philox, init_params  # noqa: F401
from .flops import flops_per_token, mfu  # noqa: F401
from . import modern  # noqa: F401
from .schedule import lr_at, train  # noqa: F401
