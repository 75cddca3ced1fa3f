"""Helpers shared by the GPU tests (device buffers in, NumPy out)."""

import sys

import numpy as np


def announce(msg):
    """Name the case on stdout before a GPU step, so a run that dies still
    says what it was doing."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(x, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def bf16_round(x):
    """float32 values rounded to bfloat16 (ties to even), as float32."""
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def rel_l2(a, ref):
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / d) if d > 0 else float(np.linalg.norm(a))


def load_params(model, params):
    """Write named float32 arrays into the model's master weights and
    refresh its bf16 shadow."""
    torch = torch_mod()
    for name, arr in params.items():
        model.param(name).copy_(torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda())
    model.sync_shadow()
    torch.cuda.synchronize()


def read_named(model, flat):
    out = {}
    h = host(flat)
    for name, off, shape, _ in model.table:
        n = int(np.prod(shape))
        out[name] = h[off:off + n].reshape(shape).copy()
    return out
