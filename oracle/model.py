"""Oracle model: GPT-2 forward and hand-written backward in plain NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings of the pages adopted here (each is listed with its justification in
the design notes of the repository):
  * pre-LN residual block, x + attn(ln_1(x)) then x + mlp(ln_2(x)): the
    printed Block.forward in [train-124M] §2.11 overwrites the residual; §2.13
    says the residual connections are the ``+=`` additions, §7 counts two
    residual additions per layer, and [repro-124M] calls the model Pre-Norm.
  * c_proj is applied after the heads are concatenated ([train-124M] §2.4
    lists c_attn and c_proj inside attn; the §2.12 listing omits it).
  * causal mask: key s is visible to query t iff s <= t ([train-124M] §5,
    ``is_causal=True``).
  * lm_head has no bias and shares its weight with wte ([train-124M] §4).
  * the softmax of the loss runs over every padded vocabulary column
    ([train-124M] §8.3 pads 50257 -> 50304; the logits are (B, T, vocab_size)).
  * GELU is the tanh approximation ([train-124M] §2.13); LayerNorm uses
    eps = 1e-5 with the biased variance (nn.LayerNorm defaults, §2.3).
  * targets equal to -1 are ignored and the mean divides by the number of
    valid targets ([grad-accum] "Cross-entropy averages within one micro-batch"
    divides by the targets of the call; the ignore index is the isolated
    lm_head workload's convention).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

LN_EPS = 1e-5
GELU_C = 0.044715


@dataclass(frozen=True)
class Config:
    """Model hyper-parameters ([train-124M] §2.1 GPT2Config, §2.6 MLP width)."""

    vocab_size: int
    block_size: int
    n_layer: int
    n_head: int
    n_embd: int
    mlp_hidden: int

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head


def param_specs(cfg: Config):
    """Parameter names and shapes, following the HF listing in [train-124M] §2.

    Linear weights are stored [out, in] (nn.Linear, as in the page's own
    modules, §2.4 and §2.6), so c_attn.weight is [3C, C].  lm_head is not a
    separate tensor: it is wte ([train-124M] §4, weight tying).
    """
    V, T, C, F = cfg.vocab_size, cfg.block_size, cfg.n_embd, cfg.mlp_hidden
    specs = [("transformer.wte.weight", (V, C)), ("transformer.wpe.weight", (T, C))]
    for layer in range(cfg.n_layer):
        p = f"transformer.h.{layer}."
        specs += [
            (p + "ln_1.weight", (C,)),
            (p + "ln_1.bias", (C,)),
            (p + "attn.c_attn.weight", (3 * C, C)),
            (p + "attn.c_attn.bias", (3 * C,)),
            (p + "attn.c_proj.weight", (C, C)),
            (p + "attn.c_proj.bias", (C,)),
            (p + "ln_2.weight", (C,)),
            (p + "ln_2.bias", (C,)),
            (p + "mlp.c_fc.weight", (F, C)),
            (p + "mlp.c_fc.bias", (F,)),
            (p + "mlp.c_proj.weight", (C, F)),
            (p + "mlp.c_proj.bias", (C,)),
        ]
    specs += [("transformer.ln_f.weight", (C,)), ("transformer.ln_f.bias", (C,))]
    return specs


def n_params(cfg: Config) -> int:
    return int(sum(np.prod(s) for _, s in param_specs(cfg)))


def is_decayed(shape) -> bool:
    """Weight decay applies to tensors with dim >= 2 only ([train-124M] §6,
    configure_optimizers)."""
    return len(shape) >= 2


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------

def gelu_tanh(u):
    """GELU, tanh approximation ([train-124M] §2.13):
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    k = float(np.sqrt(2.0 / np.pi))
    return 0.5 * u * (1.0 + np.tanh(k * (u + GELU_C * u * u * u)))


def gelu_tanh_grad(u):
    """d/du of gelu_tanh, by the product and chain rules."""
    k = float(np.sqrt(2.0 / np.pi))
    inner = k * (u + GELU_C * u * u * u)
    th = np.tanh(inner)
    dinner = k * (1.0 + 3.0 * GELU_C * u * u)
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * dinner


def layernorm_fwd(x, w, b, eps=LN_EPS):
    """LayerNorm over the last axis ([train-124M] §2.3 nn.LayerNorm(n_embd)).

    Returns y and the cache (xhat, rstd) the backward needs."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = xc * rstd
    return xhat * w + b, (xhat, rstd)


def layernorm_bwd(dy, cache, w):
    """Backward of layernorm_fwd.  dx = rstd (g - mean(g) - xhat mean(g xhat))
    with g = dy * w; dw = sum over rows of dy xhat; db = sum over rows of dy."""
    xhat, rstd = cache
    rows = dy.reshape(-1, dy.shape[-1])
    xh = xhat.reshape(-1, xhat.shape[-1])
    dw = (rows * xh).sum(axis=0)
    db = rows.sum(axis=0)
    g = dy * w
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, dw, db


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def packed_mask(row, eot):
    """Document mask of one packed row ([zero2front] "Document boundaries,
    packing and masking": attention made block-diagonal over the documents
    of a window, position ids restarted at each document).

    A document begins at its EOT token (the pipeline puts one before every
    document); tokens before the row's first EOT are the tail of a document
    cut by the window and begin at position 0.  start[t] is the last EOT
    position at or before t (0 if none); query t may attend to key s iff
    start[t] <= s <= t; pos[t] = t - start[t].
    Returns (mask [T, T] bool, pos [T] int)."""
    T = row.shape[0]
    start = np.zeros(T, dtype=np.int64)
    cur = 0
    for t in range(T):
        if row[t] == eot:
            cur = t
        start[t] = cur
    keys = np.arange(T)
    mask = (keys[None, :] <= keys[:, None]) & (keys[None, :] >= start[:, None])
    return mask, keys - start


def attention_fwd(q, k, v, mask=None):
    """Causal softmax attention for one (batch, head): q, k, v are [T, hd].

    S = q k^T / sqrt(hd), S[t, s] = -inf for s > t, P = softmax over s,
    o = P v ([train-124M] §2.12 and §5).  ``mask`` ([T, T] bool, True where
    query t may see key s) replaces the causal mask, e.g. by packed_mask's
    document mask.  Returns o and P."""
    T, hd = q.shape
    s = (q @ k.T) / np.sqrt(hd)
    if mask is None:
        hidden = np.triu(np.ones((T, T), dtype=bool), k=1)
    else:
        hidden = ~mask
    s = np.where(hidden, -np.inf, s)
    smax = s.max(axis=-1, keepdims=True)
    e = np.exp(s - smax)
    p = e / e.sum(axis=-1, keepdims=True)
    return p @ v, p


def attention_bwd(do, q, k, v, p):
    """Backward of attention_fwd for one (batch, head).

    dP = dO v^T, dv = P^T dO, dS = P (dP - rowsum(dP P)), dq = dS k / sqrt(hd),
    dk = dS^T q / sqrt(hd)."""
    hd = q.shape[1]
    dp = do @ v.T
    dv = p.T @ do
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = (ds @ k) / np.sqrt(hd)
    dk = (ds.T @ q) / np.sqrt(hd)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# loss
# ----------------------------------------------------------------------------

def cross_entropy_fwd_bwd(logits, targets, n_valid, scale, ignore_index=-1):
    """Cross-entropy rows ([train-124M] §4): softmax, pick the target, -log.

    Returns per-row losses (0 for ignored rows) and dlogits of
    scale * (sum of valid row losses) / n_valid.  Rows whose target equals
    ``ignore_index`` are ignored (the documented ``ignore_index`` of the
    library cross-entropy the pages call; -1 for the isolated lm_head
    workload); every other target must lie in [0, V)."""
    valid = targets != ignore_index
    if np.any(valid & ((targets < 0) | (targets >= logits.shape[-1]))):
        raise ValueError("target outside [0, V) that is not ignore_index")
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    se = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(se))[:, 0]
    tsafe = np.where(valid, targets, 0)
    zt = logits[np.arange(logits.shape[0]), tsafe]
    row_loss = np.where(valid, lse - zt, 0.0).astype(logits.dtype)
    prob = e / se
    dlogits = prob
    dlogits[np.arange(logits.shape[0]), tsafe] -= 1.0
    dlogits *= np.where(valid, scale / max(n_valid, 1), 0.0).astype(logits.dtype)[:, None]
    return row_loss, dlogits


def lmhead_ce(hidden, weight, targets, chunk=1024, ignore_index=-1):
    """Tied lm_head + mean cross-entropy, forward and backward, for the
    isolated lm_head workload: logits = hidden @ weight^T (no bias), loss =
    mean over valid targets (those not equal to ``ignore_index``), dHidden
    and dWeight of that mean.

    Rows are processed in chunks so the dense logits never exceed
    chunk x V; the arithmetic is the dense definition.
    Returns (loss, row_loss, dhidden, dweight)."""
    M = hidden.shape[0]
    n_valid = int((targets != ignore_index).sum())
    dhidden = np.zeros_like(hidden)
    dweight = np.zeros_like(weight)
    row_loss = np.zeros(M, dtype=hidden.dtype)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        logits = hidden[r0:r1] @ weight.T
        rl, dl = cross_entropy_fwd_bwd(logits, targets[r0:r1], n_valid, 1.0, ignore_index)
        row_loss[r0:r1] = rl
        dhidden[r0:r1] = dl @ weight
        dweight += dl.T @ hidden[r0:r1]
    loss = row_loss.astype(np.float64).sum() / n_valid if n_valid > 0 else float("nan")
    return loss, row_loss, dhidden, dweight


def lmhead_ce_sampled(hidden, weight, targets, rows, cols, chunk=1024, ignore_index=-1):
    """lmhead_ce restricted to what a large case can afford: the loss and
    per-row losses over all M rows, the rows ``rows`` of dHidden and the rows
    ``cols`` of dWeight (vocabulary entries).  Same arithmetic as lmhead_ce,
    chunk by chunk; only the requested slices of the two gradients are
    formed.  Returns (loss, row_loss, dhidden[rows], dweight[cols])."""
    M = hidden.shape[0]
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    n_valid = int((targets != ignore_index).sum())
    row_loss = np.zeros(M, dtype=hidden.dtype)
    dh = np.zeros((len(rows), hidden.shape[1]), dtype=hidden.dtype)
    dw = np.zeros((len(cols), weight.shape[1]), dtype=weight.dtype)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        logits = hidden[r0:r1] @ weight.T
        rl, dl = cross_entropy_fwd_bwd(logits, targets[r0:r1], n_valid, 1.0, ignore_index)
        row_loss[r0:r1] = rl
        here = np.nonzero((rows >= r0) & (rows < r1))[0]
        if len(here):
            dh[here] = dl[rows[here] - r0] @ weight
        dw += dl[:, cols].T @ hidden[r0:r1]
    loss = row_loss.astype(np.float64).sum() / n_valid if n_valid > 0 else float("nan")
    return loss, row_loss, dh, dw


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

def _split_heads(x, n_head):
    B, T, C = x.shape
    return x.reshape(B, T, n_head, C // n_head).transpose(0, 2, 1, 3)


def _merge_heads(x):
    B, H, T, hd = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, T, H * hd)


def packed_rows(idx, eot):
    """packed_mask of every row: (masks [B, T, T], pos [B, T]), or (None,
    positions 0..T-1 in every row) when eot is None."""
    B, T = idx.shape
    if eot is None:
        return None, np.broadcast_to(np.arange(T), (B, T))
    masks = np.empty((B, T, T), dtype=bool)
    pos = np.empty((B, T), dtype=np.int64)
    for b in range(B):
        masks[b], pos[b] = packed_mask(idx[b], eot)
    return masks, pos


def embedding_bwd(idx, dh, V, T, pos=None):
    """Gradients of x = wte[idx] + wpe[pos] ([train-124M] §2.2, §2.10) for
    dh = dL/dx [B, T, C]: (dwte [V, C], dwpe [T, C]).  Every table row
    collects the rows dh of the tokens that read it: wte by token id, wpe by
    position (0..T-1 in every row, or ``pos`` [B, T] restarted at document
    starts)."""
    C = dh.shape[-1]
    rows = dh.reshape(-1, C)
    dwte = np.zeros((V, C), dtype=dh.dtype)
    np.add.at(dwte, idx.reshape(-1), rows)
    if pos is None:
        dwpe = np.zeros((T, C), dtype=dh.dtype)
        dwpe[:idx.shape[1]] = dh.sum(axis=0)
    else:
        dwpe = np.zeros((T, C), dtype=dh.dtype)
        np.add.at(dwpe, pos.reshape(-1), rows)
    return dwte, dwpe


def forward(cfg: Config, params, idx, targets, scale=1.0, chunk=1024, want_logits=False, n_valid=None, eot=None):
    """Forward pass with every activation the backward needs.

    idx, targets: int [B, T].  Position ids are 0..T-1 in every row
    ([train-124M] §2.10).  With ``eot`` set, every row is a packed window
    under the document mask of packed_mask, positions restarted at each
    document ([zero2front] "Document boundaries, packing and masking").
    Returns (loss, row_loss [B*T], cache)."""
    B, T = idx.shape
    H, L = cfg.n_head, cfg.n_layer
    wte = params["transformer.wte.weight"]
    wpe = params["transformer.wpe.weight"]
    dt = wte.dtype
    if idx.min() < 0 or idx.max() >= cfg.vocab_size:
        raise ValueError("token id out of range")
    if T > cfg.block_size:
        raise ValueError("T exceeds block_size")

    # token + position embedding ([train-124M] §2.2, §2.10)
    masks, pos = packed_rows(idx, eot)
    h = wte[idx] + wpe[pos]
    cache = {"idx": idx, "targets": targets, "layers": [], "pos": None if eot is None else pos}
    for layer in range(L):
        p = f"transformer.h.{layer}."
        lc = {"h_in": h}
        a1, lc["ln1"] = layernorm_fwd(h, params[p + "ln_1.weight"], params[p + "ln_1.bias"])
        lc["a1"] = a1
        qkv = a1 @ params[p + "attn.c_attn.weight"].T + params[p + "attn.c_attn.bias"]
        C = cfg.n_embd
        q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
        qh, kh, vh = _split_heads(q, H), _split_heads(k, H), _split_heads(v, H)
        oh = np.empty_like(qh)
        ps = np.empty((B, H, T, T), dtype=dt)
        for b in range(B):
            for j in range(H):
                oh[b, j], ps[b, j] = attention_fwd(qh[b, j], kh[b, j], vh[b, j], None if masks is None else masks[b])
        y = _merge_heads(oh)
        lc.update(qh=qh, kh=kh, vh=vh, p=ps, y=y)
        h = h + (y @ params[p + "attn.c_proj.weight"].T + params[p + "attn.c_proj.bias"])
        lc["h_mid"] = h
        a2, lc["ln2"] = layernorm_fwd(h, params[p + "ln_2.weight"], params[p + "ln_2.bias"])
        lc["a2"] = a2
        u = a2 @ params[p + "mlp.c_fc.weight"].T + params[p + "mlp.c_fc.bias"]
        g = gelu_tanh(u)
        lc.update(u=u, g=g)
        h = h + (g @ params[p + "mlp.c_proj.weight"].T + params[p + "mlp.c_proj.bias"])
        cache["layers"].append(lc)

    z, cache["lnf"] = layernorm_fwd(h, params["transformer.ln_f.weight"], params["transformer.ln_f.bias"])
    cache["z"] = z
    zf = z.reshape(B * T, -1)
    tf = targets.reshape(B * T)
    if n_valid is None:
        n_valid = int((tf >= 0).sum())
    cache["n_valid"] = n_valid

    # tied lm_head + cross-entropy in row chunks ([train-124M] §4)
    row_loss = np.zeros(B * T, dtype=dt)
    dz = np.zeros_like(zf)
    dwte_head = np.zeros_like(wte)
    logits_all = np.empty((B * T, wte.shape[0]), dtype=dt) if want_logits else None
    for r0 in range(0, B * T, chunk):
        r1 = min(B * T, r0 + chunk)
        logits = zf[r0:r1] @ wte.T
        if want_logits:
            logits_all[r0:r1] = logits
        rl, dl = cross_entropy_fwd_bwd(logits, tf[r0:r1], n_valid, scale)
        row_loss[r0:r1] = rl
        dz[r0:r1] = dl @ wte
        dwte_head += dl.T @ zf[r0:r1]
    cache["dz"] = dz.reshape(B, T, -1)
    cache["dwte_head"] = dwte_head
    cache["logits"] = logits_all
    loss = row_loss.astype(np.float64).sum() / n_valid if n_valid > 0 else float("nan")
    return loss, row_loss, cache


def backward(cfg: Config, params, cache):
    """Hand-written backward of forward(); the loss scale and 1/n_valid are
    already folded into cache['dz'] and cache['dwte_head'].  Returns a dict of
    gradients keyed like params."""
    H, L = cfg.n_head, cfg.n_layer
    grads = {name: np.zeros_like(params[name]) for name, _ in param_specs(cfg)}
    grads["transformer.wte.weight"] += cache["dwte_head"]

    dh, dw, db = layernorm_bwd(cache["dz"], cache["lnf"], params["transformer.ln_f.weight"])
    grads["transformer.ln_f.weight"] += dw
    grads["transformer.ln_f.bias"] += db

    for layer in reversed(range(L)):
        p = f"transformer.h.{layer}."
        lc = cache["layers"][layer]
        C = cfg.n_embd
        # MLP branch: h_out = h_mid + g Wmp^T + bmp
        dflat = dh.reshape(-1, C)
        gflat = lc["g"].reshape(-1, lc["g"].shape[-1])
        grads[p + "mlp.c_proj.weight"] += dflat.T @ gflat
        grads[p + "mlp.c_proj.bias"] += dflat.sum(axis=0)
        dg = dh @ params[p + "mlp.c_proj.weight"]
        du = dg * gelu_tanh_grad(lc["u"])
        duflat = du.reshape(-1, du.shape[-1])
        grads[p + "mlp.c_fc.weight"] += duflat.T @ lc["a2"].reshape(-1, C)
        grads[p + "mlp.c_fc.bias"] += duflat.sum(axis=0)
        da2 = du @ params[p + "mlp.c_fc.weight"]
        dx, dw, db = layernorm_bwd(da2, lc["ln2"], params[p + "ln_2.weight"])
        grads[p + "ln_2.weight"] += dw
        grads[p + "ln_2.bias"] += db
        dh = dh + dx
        # attention branch: h_mid = h_in + y Wo^T + bo
        dflat = dh.reshape(-1, C)
        grads[p + "attn.c_proj.weight"] += dflat.T @ lc["y"].reshape(-1, C)
        grads[p + "attn.c_proj.bias"] += dflat.sum(axis=0)
        dy = dh @ params[p + "attn.c_proj.weight"]
        doh = _split_heads(dy, H)
        dqh = np.empty_like(doh)
        dkh = np.empty_like(doh)
        dvh = np.empty_like(doh)
        B = doh.shape[0]
        for b in range(B):
            for j in range(H):
                dqh[b, j], dkh[b, j], dvh[b, j] = attention_bwd(
                    doh[b, j], lc["qh"][b, j], lc["kh"][b, j], lc["vh"][b, j], lc["p"][b, j])
        dqkv = np.concatenate([_merge_heads(dqh), _merge_heads(dkh), _merge_heads(dvh)], axis=-1)
        dqflat = dqkv.reshape(-1, 3 * C)
        grads[p + "attn.c_attn.weight"] += dqflat.T @ lc["a1"].reshape(-1, C)
        grads[p + "attn.c_attn.bias"] += dqflat.sum(axis=0)
        da1 = dqkv @ params[p + "attn.c_attn.weight"]
        dx, dw, db = layernorm_bwd(da1, lc["ln1"], params[p + "ln_1.weight"])
        grads[p + "ln_1.weight"] += dw
        grads[p + "ln_1.bias"] += db
        dh = dh + dx

    # embeddings: wte receives the scattered rows on top of its lm_head part
    # (the tied weight, [train-124M] §4); wpe sums over the batch, or, with
    # restarted positions, over every token at each position.
    dwte, dwpe = embedding_bwd(cache["idx"], dh, cfg.vocab_size, cfg.block_size, cache["pos"])
    grads["transformer.wte.weight"] += dwte
    grads["transformer.wpe.weight"] += dwpe
    return grads


def fwd_bwd(cfg: Config, params, idx, targets, scale=1.0, grads=None, chunk=1024, n_valid=None, eot=None):
    """One micro-step: loss of the micro-batch (unscaled mean over its valid
    targets) and the gradient of scale * loss added into ``grads``
    ([train-124M] §8.1: loss / grad_accum_steps, then backward).  ``eot``
    selects the packed document mask (forward()).

    Returns (loss, row_loss, grads)."""
    loss, row_loss, cache = forward(cfg, params, idx, targets, scale=scale, chunk=chunk, n_valid=n_valid, eot=eot)
    g = backward(cfg, params, cache)
    if cache["n_valid"] == 0:
        g = {k: np.zeros_like(v) for k, v in g.items()}
    if grads is None:
        return loss, row_loss, g
    for k in grads:
        grads[k] += g[k]
    return loss, row_loss, grads
