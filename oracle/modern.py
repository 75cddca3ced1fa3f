"""Oracle for the modern GPT-2 124M variant: forward and hand-written backward
in plain NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The variant is the one [repro-124M] trains on one H100 (its model listing
and its list of training improvements): no learned position table (the
listing's ModuleDict holds only wte, the blocks and ln_f), ln_f and the block
norms are RMSNorm, rotary position embedding on q and k "implemented with
rotate_half" (x * cos + rotate_half(x) * sin), and a SwiGLU feed-forward.
[fast-1gpu] ("Step 2: the attention kernel", "Step 3: torch.compile") runs
the same three pieces (RMSNorm, RoPE, the SwiGLU gate) in its 88M model.

Readings where the pages are silent (listed with the others in the
repository's design notes):
  * RMSNorm (nn.RMSNorm with its defaults, as in the listing): y = x / sqrt(
    mean(x^2) + eps) * w, weight only, eps = float32 machine epsilon (the
    default eps of nn.RMSNorm for a float32 input; the residual stream is
    float32).
  * RoPE: the published rotary embedding (Su et al., "RoFormer", 2021) in
    the rotate_half form the page names: dimension i of a head is paired
    with dimension i + hd/2, rotate_half(x) = (-x[hd/2:], x[:hd/2]),
    angle(t, i) = t * base^(-2 i / hd) for i < hd/2 (repeated over both
    halves), base 10000, positions t = 0..T-1 of each sequence; applied to
    q and k of every head after the c_attn projection.
  * SwiGLU: the published definition (Shazeer, "GLU Variants Improve
    Transformer", 2020): FFN(x) = (silu(x W_gate^T) * (x W_up^T)) W_down^T
    with silu(g) = g * sigmoid(g); hidden width 2048 (the variant's
    configuration).  W_gate and W_up are stored as one [2F, C] tensor
    mlp.c_fc.weight: rows 0..F-1 are W_gate, rows F..2F-1 are W_up.
  * no biases anywhere (the listing's lm_head bias is not tied and is read
    as an oversight, as for the GPT-2 model; the pages give no biases for
    the new pieces).  lm_head is tied to wte.
  * init as for GPT-2 ([train-124M] §7; the same _init_weights on
    [repro-124M]): Linear weights and wte ~ N(0, 0.02), the residual
    projections attn.c_proj and mlp.c_proj ~ N(0, 0.02 (2 n_layer)^-1/2),
    RMSNorm weights 1.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .model import _merge_heads, _split_heads, attention_bwd, attention_fwd, cross_entropy_fwd_bwd, packed_rows

RMS_EPS = float(np.finfo(np.float32).eps)
ROPE_BASE = 10000.0


@dataclass(frozen=True)
class ModernConfig:
    """Hyper-parameters of the modern variant (12 layers, C = 768, 12 heads,
    SwiGLU hidden 2048, vocabulary 50304 in the full size)."""

    vocab_size: int
    block_size: int
    n_layer: int
    n_head: int
    n_embd: int
    mlp_hidden: int
    rope_base: float = ROPE_BASE
    n_kv_head: int = 0  # key/value heads (grouped-query attention); 0: one per query head

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def kv_heads(self) -> int:
        return self.n_kv_head or self.n_head

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim


def param_specs(cfg: ModernConfig):
    """Names and shapes, in the order of the module listing (wte, the blocks,
    ln_f).  Linear weights are [out, in]; lm_head is wte.  c_attn stacks the
    q rows (C), then the k and the v rows (kv_dim each: fewer than C with
    grouped-query attention)."""
    V, C, F = cfg.vocab_size, cfg.n_embd, cfg.mlp_hidden
    specs = [("transformer.wte.weight", (V, C))]
    for layer in range(cfg.n_layer):
        p = f"transformer.h.{layer}."
        specs += [
            (p + "ln_1.weight", (C,)),
            (p + "attn.c_attn.weight", (C + 2 * cfg.kv_dim, C)),
            (p + "attn.c_proj.weight", (C, C)),
            (p + "ln_2.weight", (C,)),
            (p + "mlp.c_fc.weight", (2 * F, C)),
            (p + "mlp.c_proj.weight", (C, F)),
        ]
    specs += [("transformer.ln_f.weight", (C,))]
    return specs


def n_params(cfg: ModernConfig) -> int:
    return int(sum(np.prod(s) for _, s in param_specs(cfg)))


def init_std(cfg: ModernConfig, name: str, shape) -> float:
    """Standard deviation of the N(0, std) init of one tensor (0 for the
    RMSNorm weights, which start at 1)."""
    if len(shape) == 1:
        return 0.0
    if name.endswith("attn.c_proj.weight") or name.endswith("mlp.c_proj.weight"):
        return 0.02 * (2 * cfg.n_layer) ** -0.5
    return 0.02


# ----------------------------------------------------------------------------
# pieces
# ----------------------------------------------------------------------------

def rmsnorm_fwd(x, w, eps=RMS_EPS):
    """y = x rstd w with rstd = (mean over the last axis of x^2 + eps)^-1/2.
    Returns y and the cache (xhat, rstd)."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(ms + eps)
    xhat = x * rstd
    return xhat * w, (xhat, rstd)


def rmsnorm_bwd(dy, cache, w):
    """Backward of rmsnorm_fwd: with g = dy w, dx = rstd (g - xhat mean(g xhat))
    (the chain rule through rstd: d rstd / dx = -rstd^3 x / C); dw = sum over
    rows of dy xhat."""
    xhat, rstd = cache
    dw = (dy * xhat).reshape(-1, dy.shape[-1]).sum(axis=0)
    g = dy * w
    dx = rstd * (g - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, dw


def rope_tables(T: int, hd: int, base: float = ROPE_BASE, dtype=np.float64):
    """cos and sin [T, hd] of angle(t, i) = t base^(-2i/hd), i = d mod hd/2."""
    half = hd // 2
    inv_freq = base ** (-(2.0 * np.arange(half)) / hd)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rotate_half(x):
    """(x1, x2) -> (-x2, x1) over the two halves of the last axis."""
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., half:], x[..., :half]], axis=-1)


def rope_fwd(x, cos, sin):
    """x [..., T, hd] -> x cos + rotate_half(x) sin (the page's form)."""
    return x * cos + rotate_half(x) * sin


def rope_bwd(dy, cos, sin):
    """Transpose of rope_fwd: rotate_half is the linear map (x1, x2) ->
    (-x2, x1), whose transpose is (z1, z2) -> (z2, -z1)."""
    z = dy * sin
    half = z.shape[-1] // 2
    return dy * cos + np.concatenate([z[..., half:], -z[..., :half]], axis=-1)


def silu(g):
    return g / (1.0 + np.exp(-g))


def silu_grad(g):
    """d/dg of g sigmoid(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))."""
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

def forward(cfg: ModernConfig, params, idx, targets, scale=1.0, chunk=1024, n_valid=None, eot=None, restart=True):
    """Forward pass with every activation the backward needs; idx, targets
    int [B, T].  With ``eot`` set, every row is a packed window under the
    document mask ([zero2front] "Document boundaries, packing and masking");
    ``restart`` rotates q and k by the restarted positions (else by 0..T-1,
    which the page says gives the same scores once the mask keeps documents
    apart).  With grouped-query attention (n_kv_head < n_head) query head j
    attends with key/value head j // (n_head / n_kv_head), each key/value head
    serving a run of consecutive query heads ([fast-1gpu] "Step 2: the
    attention kernel": repeat_interleave of the key and value heads).
    Returns (loss, row_loss [B*T], cache)."""
    B, T = idx.shape
    H, L, C, F = cfg.n_head, cfg.n_layer, cfg.n_embd, cfg.mlp_hidden
    hd, Hkv, Ckv = cfg.head_dim, cfg.kv_heads, cfg.kv_dim
    if H % Hkv:
        raise ValueError("n_head must be a multiple of n_kv_head")
    grp = H // Hkv
    wte = params["transformer.wte.weight"]
    dt = wte.dtype
    if idx.min() < 0 or idx.max() >= cfg.vocab_size:
        raise ValueError("token id out of range")
    if T > cfg.block_size:
        raise ValueError("T exceeds block_size")
    cos, sin = rope_tables(T, hd, cfg.rope_base, dtype=dt)
    masks, pos = packed_rows(idx, eot)
    if eot is not None and restart:
        cos, sin = cos[pos][:, None], sin[pos][:, None]  # [B, 1, T, hd]: per row, shared by the heads

    h = wte[idx]
    cache = {"idx": idx, "targets": targets, "layers": [], "cos": cos, "sin": sin}
    for layer in range(L):
        p = f"transformer.h.{layer}."
        lc = {}
        a1, lc["n1"] = rmsnorm_fwd(h, params[p + "ln_1.weight"])
        lc["a1"] = a1
        qkv = a1 @ params[p + "attn.c_attn.weight"].T
        q, k, v = qkv[..., :C], qkv[..., C:C + Ckv], qkv[..., C + Ckv:]
        qh = rope_fwd(_split_heads(q, H), cos, sin)
        kh = rope_fwd(_split_heads(k, Hkv), cos, sin)
        vh = _split_heads(v, Hkv)
        oh = np.empty_like(qh)
        ps = np.empty((B, H, T, T), dtype=dt)
        for b in range(B):
            for j in range(H):
                oh[b, j], ps[b, j] = attention_fwd(qh[b, j], kh[b, j // grp], vh[b, j // grp],
                                                   None if masks is None else masks[b])
        y = _merge_heads(oh)
        lc.update(qh=qh, kh=kh, vh=vh, p=ps, y=y)
        h = h + y @ params[p + "attn.c_proj.weight"].T
        a2, lc["n2"] = rmsnorm_fwd(h, params[p + "ln_2.weight"])
        lc["a2"] = a2
        gu = a2 @ params[p + "mlp.c_fc.weight"].T
        gate, up = gu[..., :F], gu[..., F:]
        act = silu(gate) * up
        lc.update(gate=gate, up=up, act=act)
        h = h + act @ params[p + "mlp.c_proj.weight"].T
        cache["layers"].append(lc)

    z, cache["nf"] = rmsnorm_fwd(h, params["transformer.ln_f.weight"])
    zf = z.reshape(B * T, -1)
    tf = targets.reshape(B * T)
    if n_valid is None:
        n_valid = int((tf >= 0).sum())
    cache["n_valid"] = n_valid
    row_loss = np.zeros(B * T, dtype=dt)
    dz = np.zeros_like(zf)
    dwte_head = np.zeros_like(wte)
    for r0 in range(0, B * T, chunk):
        r1 = min(B * T, r0 + chunk)
        logits = zf[r0:r1] @ wte.T
        rl, dl = cross_entropy_fwd_bwd(logits, tf[r0:r1], n_valid, scale)
        row_loss[r0:r1] = rl
        dz[r0:r1] = dl @ wte
        dwte_head += dl.T @ zf[r0:r1]
    cache["dz"] = dz.reshape(B, T, -1)
    cache["dwte_head"] = dwte_head
    loss = row_loss.astype(np.float64).sum() / n_valid if n_valid > 0 else float("nan")
    return loss, row_loss, cache


def backward(cfg: ModernConfig, params, cache):
    """Hand-written backward of forward(); the loss scale and 1/n_valid are
    folded into cache['dz'] and cache['dwte_head'].  Returns gradients keyed
    like params."""
    H, L, C, F = cfg.n_head, cfg.n_layer, cfg.n_embd, cfg.mlp_hidden
    cos, sin = cache["cos"], cache["sin"]
    grads = {name: np.zeros_like(params[name]) for name, _ in param_specs(cfg)}
    grads["transformer.wte.weight"] += cache["dwte_head"]
    dh, dw = rmsnorm_bwd(cache["dz"], cache["nf"], params["transformer.ln_f.weight"])
    grads["transformer.ln_f.weight"] += dw

    for layer in reversed(range(L)):
        p = f"transformer.h.{layer}."
        lc = cache["layers"][layer]
        # feed-forward branch: h_out = h_mid + act W_down^T
        dflat = dh.reshape(-1, C)
        grads[p + "mlp.c_proj.weight"] += dflat.T @ lc["act"].reshape(-1, F)
        dact = dh @ params[p + "mlp.c_proj.weight"]
        dgate = dact * lc["up"] * silu_grad(lc["gate"])
        dup = dact * silu(lc["gate"])
        dgu = np.concatenate([dgate, dup], axis=-1)
        grads[p + "mlp.c_fc.weight"] += dgu.reshape(-1, 2 * F).T @ lc["a2"].reshape(-1, C)
        da2 = dgu @ params[p + "mlp.c_fc.weight"]
        dx, dw = rmsnorm_bwd(da2, lc["n2"], params[p + "ln_2.weight"])
        grads[p + "ln_2.weight"] += dw
        dh = dh + dx
        # attention branch: h_mid = h_in + y W_o^T
        dflat = dh.reshape(-1, C)
        grads[p + "attn.c_proj.weight"] += dflat.T @ lc["y"].reshape(-1, C)
        dy = dh @ params[p + "attn.c_proj.weight"]
        doh = _split_heads(dy, H)
        dqh = np.empty_like(doh)
        dkh = np.zeros_like(lc["kh"])
        dvh = np.zeros_like(lc["vh"])
        B = doh.shape[0]
        grp = H // dkh.shape[1]
        for b in range(B):
            for j in range(H):
                # a key/value head shared by a group of query heads gathers
                # the gradients of all of them
                dq, dk, dv = attention_bwd(doh[b, j], lc["qh"][b, j], lc["kh"][b, j // grp], lc["vh"][b, j // grp],
                                           lc["p"][b, j])
                dqh[b, j] = dq
                dkh[b, j // grp] += dk
                dvh[b, j // grp] += dv
        # back through the rotation of q and k
        dqh = rope_bwd(dqh, cos, sin)
        dkh = rope_bwd(dkh, cos, sin)
        dqkv = np.concatenate([_merge_heads(dqh), _merge_heads(dkh), _merge_heads(dvh)], axis=-1)
        grads[p + "attn.c_attn.weight"] += dqkv.reshape(-1, dqkv.shape[-1]).T @ lc["a1"].reshape(-1, C)
        da1 = dqkv @ params[p + "attn.c_attn.weight"]
        dx, dw = rmsnorm_bwd(da1, lc["n1"], params[p + "ln_1.weight"])
        grads[p + "ln_1.weight"] += dw
        dh = dh + dx

    idx = cache["idx"]
    np.add.at(grads["transformer.wte.weight"], idx.reshape(-1), dh.reshape(-1, C))
    return grads


def fwd_bwd(cfg: ModernConfig, params, idx, targets, scale=1.0, grads=None, chunk=1024, n_valid=None, eot=None,
            restart=True):
    """One micro-step: the unscaled mean loss of the micro-batch and the
    gradient of scale * loss added into ``grads``; ``eot`` and ``restart`` as
    in forward().  Returns (loss, row_loss, grads)."""
    loss, row_loss, cache = forward(cfg, params, idx, targets, scale=scale, chunk=chunk, n_valid=n_valid, eot=eot,
                                    restart=restart)
    g = backward(cfg, params, cache)
    if cache["n_valid"] == 0:
        g = {k: np.zeros_like(v) for k, v in g.items()}
    if grads is None:
        return loss, row_loss, g
    for k in grads:
        grads[k] += g[k]
    return loss, row_loss, grads
