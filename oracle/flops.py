"""Model-FLOPs accounting.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[fast-1gpu] "MFU, defined": FLOPs per token = 6 N + 12 L H Q T, where N is the
parameter count, L the layers, H the query heads, Q the head size and T the
sequence length; MFU = tokens per second x FLOPs per token / peak FLOPS.
"""

from __future__ import annotations

from .model import Config, n_params


def flops_per_token(cfg: Config, T: int, n: int | None = None) -> int:
    N = n_params(cfg) if n is None else n
    return 6 * N + 12 * cfg.n_layer * cfg.n_head * cfg.head_dim * T


def mfu(tokens_per_s: float, flops_tok: float, peak_flops: float) -> float:
    return tokens_per_s * flops_tok / peak_flops
