"""gpt2_op_attention_bwd_noalloc (the attention backward with its per-row
buffers in the library's static per-GPU array, for callers that cannot allocate)
against gpt2_op_attention_bwd with a caller-given workspace: the same kernels
on the same inputs, so the outputs must be identical bit for bit.  Two calls
in a row, the second on a smaller input, so a stale array from the first
call would show; bf16 with the document mask and grouped key/value heads,
and float32."""

import numpy as np
import pytest

from gpu_util import announce, bf16_round, dev

pytestmark = pytest.mark.gpu


def _case(g, B, T, H, Hkv, dtype, seed, doc=False):
    import torch
    hd = 64 if dtype == "bf16" else 32
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(seed)
    width = (H + 2 * Hkv) * hd
    qkv = rng.standard_normal((B * T, width)).astype(np.float32)
    dy = rng.standard_normal((B * T, H * hd)).astype(np.float32)
    if dtype == "bf16":
        qkv, dy = bf16_round(qkv), bf16_round(dy)
    q, d = dev(qkv, td), dev(dy, td)
    seg = None
    if doc:
        tok = rng.integers(0, 50, size=(B, T)).astype(np.int32)
        tok[:, ::97] = 7
        seg = g.op_segment_starts(dev(tok), 7)
    y = torch.zeros((B * T, H * hd), dtype=td, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(q, y, lse, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    ref = torch.full((B * T, width), float("nan"), dtype=td, device="cuda")
    got = torch.full((B * T, width), float("nan"), dtype=td, device="cuda")
    g.op_attention_bwd(q, y, d, lse, ref, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    g.op_attention_bwd_noalloc(q, y, d, lse, got, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    assert torch.equal(ref, got), (B, T, H, Hkv, dtype)


def test_attention_bwd_noalloc_equals_workspace_entry():
    import torch
    import gpt_pretraining_step_amd as g
    assert torch.cuda.is_available()
    assert g.lib().gpt2_noalloc_scratch_bytes() == 8 << 20
    announce("attention bwd no-alloc: bf16 B=16 T=1024 H=12, then B=2 T=300 H=12 Hkv=4 with document mask")
    _case(g, 16, 1024, 12, 12, "bf16", 1)
    _case(g, 2, 300, 12, 4, "bf16", 2, doc=True)
    announce("attention bwd no-alloc: float32 B=3 T=100 H=4, then B=1 T=40 H=2")
    _case(g, 3, 100, 4, 4, "f32", 3)
    _case(g, 1, 40, 2, 2, "f32", 4)


def test_attention_bwd_noalloc_rejects_sizes_beyond_its_array():
    import torch
    import gpt_pretraining_step_amd as g
    announce("attention bwd no-alloc: size limit (host check, nothing launched)")
    B, T, H = 86, 1024, 12  # B * H * T = 1,056,768 > 1,048,576
    t = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(g.GPT2Error) as e:
        g.op_attention_bwd_noalloc(t, t, t, lse, t, B, T, H, 64)
    assert e.value.status == g._ffi.GPT2_ERR_SHAPE
