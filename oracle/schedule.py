"""Oracle learning-rate schedule and training loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[repro-124M] (hyper-parameter listing and the "优化训练" list) trains with a
warmed-up cosine schedule: max_lr 1.5e-3, min_lr = 0.1 max_lr, 300 warmup
steps, 19,073 steps in all; [zero2front] (the training loop) leaves the
schedule as the next step.  No page prints the formula.  The reading taken
here is the plainest one the numbers support, for optimizer step s counted
from 0:

  * warmup: the rate climbs linearly and reaches max_lr on the last warmup
    step: lr = max_lr (s + 1) / warmup for s < warmup;
  * decay: over the remaining steps the rate follows half a cosine period from
    max_lr down to min_lr: with r = (s - warmup) / (max_steps - warmup),
    lr = min_lr + (max_lr - min_lr) (1 + cos(pi r)) / 2;
  * past max_steps the rate stays at min_lr.
"""

from __future__ import annotations

import math

import numpy as np

from .optim import clip_adamw_step


def lr_at(step: int, max_lr: float, min_lr: float, warmup: int, max_steps: int) -> float:
    if step < warmup:
        return max_lr * (step + 1) / warmup
    if step > max_steps:
        return min_lr
    r = (step - warmup) / (max_steps - warmup)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + math.cos(math.pi * r))


def train(cfg, params, batches, steps, fwd_bwd, max_lr, min_lr, warmup, max_steps, beta1=0.9, beta2=0.95,
          eps=1e-8, weight_decay=0.1, max_norm=1.0):
    """The [zero2front] loop: per optimizer step, zero the gradients, run every
    micro-batch of `batches(step)` (a list of (tokens, targets)) forward and
    backward with loss / len(micro-batches), then clip + AdamW at lr_at(step).
    `params` is updated in place.  Returns [(mean micro-batch loss, pre-clip
    grad norm, lr)] per step."""
    m = {k: np.zeros_like(v) for k, v in params.items()}
    v = {k: np.zeros_like(x) for k, x in params.items()}
    out = []
    for s in range(steps):
        mbs = batches(s)
        grads = {k: np.zeros_like(x) for k, x in params.items()}
        losses = []
        for tok, tgt in mbs:
            loss = fwd_bwd(cfg, params, tok, tgt, scale=1.0 / len(mbs), grads=grads)[0]
            losses.append(float(loss))
        lr = lr_at(s, max_lr, min_lr, warmup, max_steps)
        norm = clip_adamw_step(params, grads, m, v, s + 1, lr, beta1, beta2, eps, weight_decay, max_norm)
        out.append((float(np.mean(losses)), float(norm), lr))
    return out
