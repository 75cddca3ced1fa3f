"""The training loop around the step: warmed-up cosine learning rate,
gradient accumulation, clip + AdamW, one loss / norm readback per step.

"GPT" chapter of Zero to Frontier (the training loop: zero the gradients,
accumulate loss / grad_accum_steps over the micro-batches, step the
optimizer); "Reproduce GPT-2 124M 复盘" (hyper-parameters: warmup 300 steps,
cosine decay from max_lr to 0.1 max_lr over 19,073 steps, clip 1.0, AdamW
betas (0.9, 0.95), weight decay 0.1).  Host-side orchestration only: the
learning rate comes from gpt2_lr_at and every computation from the library.
"""

from __future__ import annotations

from dataclasses import dataclass

from ._ffi import lib


@dataclass
class Schedule:
    max_lr: float = 1.5e-3
    min_lr: float = 1.5e-4
    warmup: int = 300
    max_steps: int = 19073

    def lr(self, step: int) -> float:
        return float(lib().gpt2_lr_at(step, self.max_lr, self.min_lr, self.warmup, self.max_steps))


def train(model, batches, steps: int, schedule: Schedule, beta1: float = 0.9, beta2: float = 0.95,
          eps: float = 1e-8, weight_decay: float = 0.1, max_norm: float = 1.0, graph: bool = False):
    """Run `steps` optimizer steps of `model` (a GPT2).  `batches(step)` returns
    the step's micro-batches, a list of (tokens, targets) int32 device tensors
    of one shape.  With graph=True the micro-steps replay a HIP graph captured
    over a pair of staging buffers (the micro-batches are copied into them).
    Returns [(mean micro-batch loss, pre-clip gradient norm, lr)] per step,
    read back once per step."""
    import torch
    hist = []
    stage = None
    for _ in range(steps):
        s = model.step  # optimizer steps taken so far: this step's index
        mbs = batches(s)
        ga = len(mbs)
        losses = torch.zeros(ga, dtype=torch.float32, device=mbs[0][0].device)
        model.zero_grad()
        if graph:
            if stage is None or stage[0].shape != mbs[0][0].shape or stage[2] != ga:
                tok = torch.empty_like(mbs[0][0])
                tgt = torch.empty_like(mbs[0][1])
                loss_buf = torch.zeros(1, dtype=torch.float32, device=tok.device)
                tok.copy_(mbs[0][0])
                tgt.copy_(mbs[0][1])
                # one eager micro-step at this shape sets up the library's tables;
                # its gradients are cleared again before the step runs
                model.fwd_bwd(tok, tgt, loss_scale=1.0 / ga, loss_out=loss_buf)
                model.graph_capture(tok, tgt, loss_scale=1.0 / ga, loss_out=loss_buf)
                model.zero_grad()
                stage = (tok, tgt, ga, loss_buf)
            tok, tgt, _, loss_buf = stage
            for k, (x, y) in enumerate(mbs):
                tok.copy_(x)
                tgt.copy_(y)
                model.graph_launch()
                losses[k:k + 1].copy_(loss_buf)
        else:
            for k, (x, y) in enumerate(mbs):
                model.fwd_bwd(x, y, loss_scale=1.0 / ga, loss_out=losses[k:k + 1])
        lr = schedule.lr(s)
        norm = model.clip_adamw_step(lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                                     max_norm=max_norm)
        hist.append((float(losses.mean().item()), float(norm.item()), lr))
    return hist
