"""Oracle optimizer: global-norm clipping and AdamW, written out element-wise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages call the library routines: ``clip_grad_norm_(params, 1.0)``
([repro-124M], "优化训练" list) and ``torch.optim.AdamW(..., betas=(0.9, 0.95),
eps=1e-8)`` with decay only on tensors of dim >= 2 ([train-124M] §6).  The
simplified formulas printed in [train-124M] §6 drop the bias correction and
write the decay without the learning rate; the routine the page actually calls
is the documented decoupled-decay AdamW, which is what is written here:

    p <- p (1 - lr wd)                       (decayed tensors only)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

Clipping follows the documented rule: the global L2 norm over every gradient,
coef = min(1, max_norm / (norm + 1e-6)), every gradient multiplied by coef.
The norm returned is the one before clipping.
"""

from __future__ import annotations

import math

import numpy as np

from .model import is_decayed

CLIP_EPS = 1e-6


def global_grad_norm(grads) -> float:
    """sqrt of the sum of squares of every gradient element, in float64."""
    total = 0.0
    for g in grads.values():
        g64 = np.asarray(g, dtype=np.float64)
        total += float((g64 * g64).sum())
    return math.sqrt(total)


def clip_coef(norm: float, max_norm: float) -> float:
    return min(1.0, max_norm / (norm + CLIP_EPS))


def adamw_update(p, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """One AdamW update of one tensor at step t (t counts from 1).

    Arrays are updated in place; the arithmetic runs in the arrays' dtype
    except the bias corrections, which are float64 scalars."""
    if weight_decay != 0.0:
        p *= (1.0 - lr * weight_decay)
    m *= beta1
    m += (1.0 - beta1) * g
    v *= beta2
    v += (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    mhat = m / bc1
    vhat = v / bc2
    p -= lr * mhat / (np.sqrt(vhat) + eps)


def clip_adamw_step(params, grads, m, v, t, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                    weight_decay=0.1, max_norm=1.0):
    """Clip all grads by the global norm, then AdamW every tensor.

    params, grads, m, v: dicts of arrays keyed alike (updated in place; grads
    are scaled by the clip coefficient).  t is the step number after the
    increment (1 on the first call).  Returns the pre-clip norm.  A
    non-finite norm leaves everything unchanged."""
    norm = global_grad_norm(grads)
    if not math.isfinite(norm):
        return norm
    coef = clip_coef(norm, max_norm)
    for name in params:
        g = grads[name]
        g *= coef
        wd = weight_decay if is_decayed(params[name].shape) else 0.0
        adamw_update(params[name], g, m[name], v[name], t, lr, beta1, beta2, eps, wd)
    return norm
