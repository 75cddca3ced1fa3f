"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: finite differences, closed
forms, invariants, brute-force loops, the worked examples the pages print
(tests/golden/), published known-answer vectors and the documented PyTorch
library routines on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import model as M
from oracle import optim as O
from oracle import init as I
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


TINY = M.Config(vocab_size=11, block_size=8, n_layer=2, n_head=2, n_embd=8, mlp_hidden=32)
C0 = M.Config(vocab_size=66, block_size=64, n_layer=2, n_head=4, n_embd=64, mlp_hidden=256)
GPT2 = M.Config(vocab_size=50304, block_size=1024, n_layer=12, n_head=12, n_embd=768, mlp_hidden=3072)


def tiny_params(dtype=np.float64, seed=3):
    p = synthetic.random_params(M.param_specs(TINY), seed=seed, matrix_std=0.3, vector_std=0.2)
    return {k: v.astype(dtype) for k, v in p.items()}


def tiny_batch(seed=5, B=2, T=5, ignore=()):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, TINY.vocab_size, size=(B, T))
    y = rng.integers(0, TINY.vocab_size, size=(B, T))
    for (b, t) in ignore:
        y[b, t] = -1
    return x, y


# ----------------------------------------------------------------------------
# whole model: finite differences (fp64)
# ----------------------------------------------------------------------------

def _loss(params, x, y):
    loss, _, _ = M.forward(TINY, params, x, y)
    return loss


@pytest.mark.parametrize("ignore", [(), ((0, 1), (1, 4))])
def test_finite_differences_all_tensor_kinds(ignore):
    params = tiny_params()
    x, y = tiny_batch(ignore=ignore)
    scale = 0.37
    loss, _, grads = M.fwd_bwd(TINY, params, x, y, scale=scale)
    rng = np.random.default_rng(11)
    h = 1e-6
    names = [n for n, _ in M.param_specs(TINY)]
    checked = 0
    worst = 0.0
    for name in names:
        p = params[name]
        flat = p.reshape(-1)
        k = min(flat.size, 16)
        for i in rng.choice(flat.size, size=k, replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = _loss(params, x, y)
            flat[i] = old - h
            lm = _loss(params, x, y)
            flat[i] = old
            fd = scale * (lp - lm) / (2 * h)
            an = grads[name].reshape(-1)[i]
            err = abs(fd - an) / max(abs(an), 1e-3)  # FD noise floor ~eps*L/h ~ 3e-10
            worst = max(worst, err)
            checked += 1
            assert err < 1e-6, (name, i, fd, an)
    assert checked >= 300
    # directional derivative along one random direction over every tensor
    d = {n: rng.standard_normal(params[n].shape) for n in names}
    plus = {n: params[n] + h * d[n] for n in names}
    minus = {n: params[n] - h * d[n] for n in names}
    fd = scale * (_loss(plus, x, y) - _loss(minus, x, y)) / (2 * h)
    an = sum(float((grads[n] * d[n]).sum()) for n in names)
    assert abs(fd - an) / abs(an) < 1e-6


def test_finite_differences_wte_rows_both_roles():
    """wte is used by the embedding and the tied lm_head: rows that appear
    as input ids and rows that appear only as output columns both match."""
    params = tiny_params(seed=9)
    x, y = tiny_batch(seed=2)
    _, _, grads = M.fwd_bwd(TINY, params, x, y)
    used = set(np.unique(x).tolist())
    unused = [v for v in range(TINY.vocab_size) if v not in used]
    rows = list(used)[:2] + unused[:2]
    h = 1e-6
    w = params["transformer.wte.weight"]
    for r in rows:
        for c in range(TINY.n_embd):
            old = w[r, c]
            w[r, c] = old + h
            lp = _loss(params, x, y)
            w[r, c] = old - h
            lm = _loss(params, x, y)
            w[r, c] = old
            fd = (lp - lm) / (2 * h)
            an = grads["transformer.wte.weight"][r, c]
            assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3)


# ----------------------------------------------------------------------------
# causality
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("t", [0, 2, 30, 62])
def test_causality_bitwise(t):
    params = {k: v.astype(np.float32) for k, v in synthetic.random_params(M.param_specs(C0), seed=1).items()}
    B, T = 2, 64
    rng = np.random.default_rng(4)
    x = rng.integers(0, C0.vocab_size, size=(B, T))
    y = rng.integers(0, C0.vocab_size, size=(B, T))
    _, rl1, c1 = M.forward(C0, params, x, y, want_logits=True)
    x2 = x.copy()
    x2[:, t + 1:] = rng.integers(0, C0.vocab_size, size=(B, T - t - 1))
    assert (x2 != x).any()
    _, rl2, c2 = M.forward(C0, params, x2, y, want_logits=True)
    rl1 = rl1.reshape(B, T)
    rl2 = rl2.reshape(B, T)
    lg1 = c1["logits"].reshape(B, T, -1)
    lg2 = c2["logits"].reshape(B, T, -1)
    assert np.array_equal(rl1[:, :t + 1], rl2[:, :t + 1])
    assert np.array_equal(lg1[:, :t + 1], lg2[:, :t + 1])
    assert not np.array_equal(lg1[:, t + 1:], lg2[:, t + 1:])


# ----------------------------------------------------------------------------
# initial loss ~ ln V ([train-124M] §7)
# ----------------------------------------------------------------------------

def test_initial_loss_c0():
    params = I.init_params(C0, seed=42)
    stream = synthetic.uniform_stream(4 * 64 + 1, C0.vocab_size, seed=1337)
    x, y = synthetic.micro_batch(stream, 0, 4, 64)
    loss, _, _ = M.forward(C0, params, x, y)
    assert abs(loss - math.log(66)) <= 0.1
    # second-order estimate ln V + C * 0.02^2 / 2
    assert abs(loss - (math.log(66) + 0.5 * 64 * 0.02 ** 2)) <= 0.05


@pytest.mark.slow
def test_initial_loss_gpt2_124m():
    params = I.init_params(GPT2, seed=42)
    stream = synthetic.token_stream(2 * 128 + 1)
    x, y = synthetic.micro_batch(stream, 0, 2, 128)
    loss, _, _ = M.forward(GPT2, params, x, y)
    assert abs(loss - math.log(50257)) <= 0.3
    assert abs(loss - 10.98) <= 0.15


# ----------------------------------------------------------------------------
# gradient accumulation identity ([grad-accum]; [train-124M] §8.1)
# ----------------------------------------------------------------------------

def _c0_params64():
    return {k: v.astype(np.float64) for k, v in synthetic.random_params(M.param_specs(C0), seed=8).items()}


def test_accumulation_identity_equal_counts():
    params = _c0_params64()
    stream = synthetic.uniform_stream(4 * 64 + 1, C0.vocab_size, seed=21)
    x, y = synthetic.micro_batch(stream, 0, 4, 64)
    acc = {n: np.zeros(s) for n, s in M.param_specs(C0)}
    losses = []
    for g in range(4):
        l, _, acc = M.fwd_bwd(C0, params, x[g:g + 1], y[g:g + 1], scale=0.25, grads=acc)
        losses.append(l)
    lu, _, gu = M.fwd_bwd(C0, params, x, y, scale=1.0)
    assert abs(sum(losses) / 4 - lu) <= 1e-12 * abs(lu)
    for n in gu:
        denom = np.linalg.norm(gu[n])
        if denom > 0:
            assert np.linalg.norm(acc[n] - gu[n]) / denom <= 1e-6, n


def test_accumulation_identity_fails_with_unequal_counts_by_predicted_amount():
    params = _c0_params64()
    stream = synthetic.uniform_stream(2 * 64 + 1, C0.vocab_size, seed=22)
    x, y = synthetic.micro_batch(stream, 0, 2, 64)
    y = y.copy()
    y[1, 10:] = -1  # micro-batch 1 keeps 10 of 64 targets
    n = [int((y[g] >= 0).sum()) for g in range(2)]
    per = [M.fwd_bwd(C0, params, x[g:g + 1], y[g:g + 1], scale=1.0) for g in range(2)]
    acc = {k: 0.5 * per[0][2][k] + 0.5 * per[1][2][k] for k in per[0][2]}
    lu, _, gu = M.fwd_bwd(C0, params, x, y, scale=1.0)
    # union mean weights each micro-batch by its valid count
    pred = {k: (n[0] * per[0][2][k] + n[1] * per[1][2][k]) / (n[0] + n[1]) for k in gu}
    assert abs(lu - (n[0] * per[0][0] + n[1] * per[1][0]) / (n[0] + n[1])) <= 1e-12
    w = gu["transformer.h.0.mlp.c_fc.weight"]
    assert np.linalg.norm(pred["transformer.h.0.mlp.c_fc.weight"] - w) <= 1e-10 * np.linalg.norm(w)
    # the naive 1/G accumulation is off by the predicted difference
    diff = acc["transformer.h.0.mlp.c_fc.weight"] - w
    pdiff = (0.5 - n[0] / sum(n)) * per[0][2]["transformer.h.0.mlp.c_fc.weight"] + \
            (0.5 - n[1] / sum(n)) * per[1][2]["transformer.h.0.mlp.c_fc.weight"]
    assert np.linalg.norm(diff) > 1e-2 * np.linalg.norm(w)
    assert np.linalg.norm(diff - pdiff) <= 1e-10 * np.linalg.norm(w)


def _logits_with_losses(losses, V=4):
    """Rows of logits whose cross-entropy with target 0 equals the given
    losses: z = (0, c, c, ...) gives lse - 0 = log(1 + (V-1) e^c)."""
    rows = []
    for L in losses:
        c = math.log((math.exp(L) - 1.0) / (V - 1))
        rows.append([0.0] + [c] * (V - 1))
    return np.array(rows, dtype=np.float64)


def test_grad_accum_worked_example_through_cross_entropy():
    g = golden("grad_accum_worked_example.json")
    objectives = []
    for rank in ("rank0", "rank1"):
        micro = g[rank + "_token_losses"]
        means = []
        scaled = 0.0
        for toks in micro:
            logits = _logits_with_losses(toks)
            targets = np.zeros(len(toks), dtype=np.int64)
            rl, _ = M.cross_entropy_fwd_bwd(logits, targets, len(toks), 1.0)
            means.append(rl.sum() / len(toks))
            scaled += rl.sum() / len(toks) / len(micro)
        np.testing.assert_allclose(means, g[rank + "_micro_means"], rtol=1e-12)
        np.testing.assert_allclose(scaled, g[rank + "_objective"], rtol=1e-12)
        objectives.append(scaled)
    np.testing.assert_allclose(sum(objectives) / 2, g["ddp_average"], rtol=1e-12)
    allt = [v for r in ("rank0", "rank1") for mb in g[r + "_token_losses"] for v in mb]
    logits = _logits_with_losses(allt)
    rl, _ = M.cross_entropy_fwd_bwd(logits, np.zeros(8, dtype=np.int64), 8, 1.0)
    np.testing.assert_allclose(rl.sum() / 8, g["eight_token_mean"], rtol=1e-12)


# ----------------------------------------------------------------------------
# cross-entropy
# ----------------------------------------------------------------------------

def test_ce_zero_hidden_special_case():
    rng = np.random.default_rng(0)
    V, C, Mr = 50304, 16, 6
    W = rng.standard_normal((V, C))
    h = np.zeros((Mr, C))
    tg = rng.integers(0, 50257, size=Mr)
    tg[2] = -1
    loss, rl, dh, dw = M.lmhead_ce(h, W, tg)
    assert loss == pytest.approx(math.log(50304), abs=1e-12)
    nv = Mr - 1
    for i in range(Mr):
        if tg[i] < 0:
            assert np.all(dh[i] == 0)
        else:
            np.testing.assert_allclose(dh[i], (W.mean(axis=0) - W[tg[i]]) / nv, rtol=1e-9, atol=1e-15)


def test_ce_brute_force_and_invariants():
    rng = np.random.default_rng(1)
    Mr, C, V = 7, 5, 9
    h = rng.standard_normal((Mr, C))
    W = rng.standard_normal((V, C))
    tg = rng.integers(0, V, size=Mr)
    tg[3] = -1
    loss, rl, dh, dw = M.lmhead_ce(h, W, tg, chunk=3)
    nv = Mr - 1
    # brute force: per-element loops
    bl = 0.0
    bdh = np.zeros_like(h)
    bdw = np.zeros_like(W)
    for i in range(Mr):
        if tg[i] < 0:
            continue
        z = [sum(h[i, c] * W[v, c] for c in range(C)) for v in range(V)]
        mz = max(z)
        se = sum(math.exp(zz - mz) for zz in z)
        bl += (mz + math.log(se) - z[tg[i]]) / nv
        for v in range(V):
            d = (math.exp(z[v] - mz) / se - (1.0 if v == tg[i] else 0.0)) / nv
            for c in range(C):
                bdh[i, c] += d * W[v, c]
                bdw[v, c] += d * h[i, c]
    assert loss == pytest.approx(bl, rel=1e-12)
    np.testing.assert_allclose(dh, bdh, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dw, bdw, rtol=1e-10, atol=1e-14)
    # each row of dlogits sums to zero, so dWeight's columns sum to zero
    np.testing.assert_allclose(dw.sum(axis=0), 0.0, atol=1e-12)
    assert np.all(dh[3] == 0)


def test_ce_ignore_index_brute_force_and_library():
    """ignore_index names the ignored target value, as in the library
    cross-entropy the pages call; a value inside [0, V) ignores that class's
    rows.  Brute force by per-element loops over the rows that count, and
    torch's CPU cross_entropy(ignore_index=...) with autograd (float64)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    Mr, C, V = 11, 4, 7
    h = rng.standard_normal((Mr, C))
    W = rng.standard_normal((V, C))
    tg = rng.integers(0, V, size=Mr)
    tg[tg == 4] = 5
    tg[[1, 6, 9]] = 4
    for ig in (4, -100):
        t2 = tg.copy()
        if ig < 0:
            t2[[1, 6, 9]] = ig
        loss, rl, dh, dw = M.lmhead_ce(h, W, t2, chunk=4, ignore_index=ig)
        keep = [i for i in range(Mr) if t2[i] != ig]
        nv = len(keep)
        assert nv == Mr - 3
        bl, bdh, bdw = 0.0, np.zeros_like(h), np.zeros_like(W)
        for i in keep:
            z = [sum(h[i, c] * W[v, c] for c in range(C)) for v in range(V)]
            mz = max(z)
            se = sum(math.exp(zz - mz) for zz in z)
            bl += (mz + math.log(se) - z[t2[i]]) / nv
            for v in range(V):
                d = (math.exp(z[v] - mz) / se - (1.0 if v == t2[i] else 0.0)) / nv
                bdh[i] += d * W[v]
                bdw[v] += d * h[i]
        assert loss == pytest.approx(bl, rel=1e-12)
        np.testing.assert_allclose(dh, bdh, rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(dw, bdw, rtol=1e-10, atol=1e-14)
        ht = torch.tensor(h, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        lt = F.cross_entropy(ht @ Wt.T, torch.tensor(t2), ignore_index=ig)
        lt.backward()
        assert float(lt) == pytest.approx(loss, rel=1e-12)
        np.testing.assert_allclose(ht.grad.numpy(), dh, rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(Wt.grad.numpy(), dw, rtol=1e-10, atol=1e-14)
    with pytest.raises(ValueError):  # a negative target other than ignore_index is not a class
        M.lmhead_ce(h, W, np.where(tg == 4, -1, tg), ignore_index=-100)


def test_ce_sampled_slices_equal_dense():
    """lmhead_ce_sampled gives the dense lmhead_ce's loss and per-row losses
    and exactly its rows / vocabulary entries of dHidden and dWeight."""
    rng = np.random.default_rng(6)
    Mr, C, V = 23, 6, 13
    h = rng.standard_normal((Mr, C))
    W = rng.standard_normal((V, C))
    tg = rng.integers(0, V, size=Mr)
    tg[[0, 5, 22]] = -1
    loss, rl, dh, dw = M.lmhead_ce(h, W, tg)
    rows, cols = np.array([0, 4, 5, 17, 22]), np.array([12, 0, 3, 3])
    for chunk in (1, 5, 1024):
        l2, rl2, dhs, dws = M.lmhead_ce_sampled(h, W, tg, rows, cols, chunk=chunk)
        assert l2 == pytest.approx(loss, rel=1e-13)
        np.testing.assert_allclose(rl2, rl, rtol=1e-13, atol=0)
        np.testing.assert_allclose(dhs, dh[rows], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dws, dw[cols], rtol=1e-12, atol=1e-15)


def test_ce_all_ignored_gives_nan_and_no_grad():
    h = np.ones((3, 4))
    W = np.ones((5, 4))
    loss, rl, dh, dw = M.lmhead_ce(h, W, np.full(3, -1))
    assert math.isnan(loss)
    assert np.all(dh == 0) and np.all(dw == 0)


# ----------------------------------------------------------------------------
# LayerNorm, attention, GELU
# ----------------------------------------------------------------------------

def test_embedding_bwd_brute_force_and_chain_rule():
    """Scatter-add of the embedding gradients: brute-force loops over every
    token (wte by id, wpe by position, restarted positions under a document
    mask), and the chain rule through x = wte[idx] + wpe[pos]: for any
    tables, sum(dh * x) = sum(dwte * wte) + sum(dwpe * wpe)."""
    rng = np.random.default_rng(11)
    B, T, C, V = 3, 9, 5, 7
    idx = rng.integers(0, V, size=(B, T))
    idx[0, 4] = 6  # an EOT id inside a row
    dh = rng.standard_normal((B, T, C))
    _, pos = M.packed_rows(idx, 6)
    for p in (None, pos):
        dwte, dwpe = M.embedding_bwd(idx, dh, V, T + 2, p)
        bw, bp = np.zeros((V, C)), np.zeros((T + 2, C))
        for b in range(B):
            for t in range(T):
                bw[idx[b, t]] += dh[b, t]
                bp[t if p is None else p[b, t]] += dh[b, t]
        np.testing.assert_allclose(dwte, bw, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dwpe, bp, rtol=0, atol=1e-12)
        wte, wpe = rng.standard_normal((V, C)), rng.standard_normal((T + 2, C))
        x = wte[idx] + wpe[np.broadcast_to(np.arange(T), (B, T)) if p is None else p]
        assert np.sum(dh * x) == pytest.approx(np.sum(dwte * wte) + np.sum(dwpe * wpe), rel=1e-12)
    assert np.all(pos[0, 4:] == np.arange(T - 4))  # the positions restart at the EOT


def test_layernorm_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 32)) * 3 + 1
    w = np.ones(32)
    b = np.zeros(32)
    y, (xhat, rstd) = M.layernorm_fwd(x, w, b)
    var = x.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=-1), var / (var + 1e-5), rtol=1e-12)
    dy = rng.standard_normal((10, 32))
    w = rng.standard_normal(32)
    _, cache = M.layernorm_fwd(x, w, b)
    dx, dw, db = M.layernorm_bwd(dy, cache, w)
    np.testing.assert_allclose(dx.sum(axis=-1), 0.0, atol=1e-12)
    # sum_i dx_i xhat_i = rstd * eps / (var + eps) * sum_i g_i xhat_i (zero when eps = 0)
    g = dy * w
    pred = cache[1][:, 0] * 1e-5 / (var + 1e-5) * (g * cache[0]).sum(axis=-1)
    np.testing.assert_allclose((dx * cache[0]).sum(axis=-1), pred, rtol=1e-6, atol=1e-14)
    _, cache0 = M.layernorm_fwd(x, w, b, eps=0.0)
    dx0, _, _ = M.layernorm_bwd(dy, cache0, w)
    np.testing.assert_allclose((dx0 * cache0[0]).sum(axis=-1), 0.0, atol=1e-11)


def test_attention_special_cases_and_brute_force():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 4)) for _ in range(3))
    o, p = M.attention_fwd(q, k, v)
    np.testing.assert_allclose(o, v, rtol=1e-15)
    T, hd = 6, 4
    q, k, v = (rng.standard_normal((T, hd)) for _ in range(3))
    o, p = M.attention_fwd(q, k, v)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-15)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=1e-14)
    assert np.all(np.triu(p, 1) == 0)
    for t in range(T):
        sc = [sum(q[t, d] * k[s, d] for d in range(hd)) / math.sqrt(hd) for s in range(t + 1)]
        mx = max(sc)
        e = [math.exp(s_ - mx) for s_ in sc]
        tot = sum(e)
        for d in range(hd):
            ref = sum(e[s] / tot * v[s, d] for s in range(t + 1))
            assert o[t, d] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_attention_key_shift_invariance():
    """Adding one vector to every key leaves each softmax row unchanged, so
    the key gradients of one head sum to zero."""
    rng = np.random.default_rng(4)
    T, hd = 9, 4
    q, k, v = (rng.standard_normal((T, hd)) for _ in range(3))
    o, p = M.attention_fwd(q, k, v)
    do = rng.standard_normal((T, hd))
    dq, dk, dv = M.attention_bwd(do, q, k, v, p)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    o2, _ = M.attention_fwd(q, k + rng.standard_normal(hd), v)
    np.testing.assert_allclose(o2, o, rtol=1e-10)


def test_model_key_bias_gradient_vanishes():
    params = tiny_params()
    x, y = tiny_batch()
    _, _, g = M.fwd_bwd(TINY, params, x, y)
    C = TINY.n_embd
    for layer in range(TINY.n_layer):
        gb = g[f"transformer.h.{layer}.attn.c_attn.bias"]
        assert np.abs(gb[C:2 * C]).max() <= 1e-12 * np.abs(gb).max() + 1e-15


def test_gelu_against_erf_form_and_derivative():
    u = np.linspace(-6, 6, 2001)
    exact = 0.5 * u * (1 + np.array([math.erf(x / math.sqrt(2)) for x in u]))
    assert np.abs(M.gelu_tanh(u) - exact).max() < 1e-3
    assert M.gelu_tanh(np.array([0.0]))[0] == 0.0
    h = 1e-6
    fd = (M.gelu_tanh(u + h) - M.gelu_tanh(u - h)) / (2 * h)
    np.testing.assert_allclose(M.gelu_tanh_grad(u), fd, rtol=1e-7, atol=1e-9)


# ----------------------------------------------------------------------------
# optimizer
# ----------------------------------------------------------------------------

def test_adamw_closed_form_first_step():
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal(1000)
    g = rng.standard_normal(1000) * 1e-2
    lr, wd, eps = 6e-4, 0.1, 1e-8
    p = p0.copy()
    m = np.zeros(1000)
    v = np.zeros(1000)
    O.adamw_update(p, g, m, v, 1, lr, 0.9, 0.95, eps, wd)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-16)
    # constant gradient: the bias-corrected moments equal g and g^2 at every step
    for t in range(2, 6):
        prev = p.copy()
        O.adamw_update(p, g, m, v, t, lr, 0.9, 0.95, eps, wd)
        np.testing.assert_allclose(p, prev * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-14)


def test_clip_identities():
    rng = np.random.default_rng(6)
    grads = {"a": rng.standard_normal((30, 4)), "b": rng.standard_normal(7)}
    norm = O.global_grad_norm(grads)
    assert norm == pytest.approx(math.sqrt(sum((g ** 2).sum() for g in grads.values())), rel=1e-14)
    for max_norm in (0.5 * norm, 2 * norm):
        c = O.clip_coef(norm, max_norm)
        clipped = {k: v * c for k, v in grads.items()}
        after = O.global_grad_norm(clipped)
        assert after == pytest.approx(min(norm, max_norm * norm / (norm + 1e-6)), rel=1e-12)
    assert O.clip_coef(norm, 2 * norm) == 1.0


def test_nonfinite_norm_skips_update():
    p = {"w": np.ones((2, 2))}
    g = {"w": np.array([[np.inf, 0], [0, 0]])}
    m = {"w": np.zeros((2, 2))}
    v = {"w": np.zeros((2, 2))}
    n = O.clip_adamw_step(p, g, m, v, 1, 1e-3)
    assert not math.isfinite(n)
    assert np.all(p["w"] == 1) and np.all(m["w"] == 0)


def test_weight_decay_split_by_dim():
    specs = M.param_specs(GPT2)
    decayed = [n for n, s in specs if M.is_decayed(s)]
    assert len(specs) == 148 and len(decayed) == 50
    assert "transformer.wte.weight" in decayed and "transformer.wpe.weight" in decayed
    assert all(not n.endswith("bias") for n in decayed)


# ----------------------------------------------------------------------------
# the pages' arithmetic
# ----------------------------------------------------------------------------

def test_mfu_worked_example():
    g = golden("mfu_worked_example.json")
    cfg = M.Config(vocab_size=1, block_size=g["seq_len"], n_layer=g["n_layer"], n_head=g["n_head"],
                   n_embd=g["n_head"] * g["head_dim"], mlp_hidden=1)
    f = oracle.flops_per_token(cfg, g["seq_len"], n=g["n_params"])
    assert f == g["flops_per_token"]
    assert round(6 * g["n_params"] / 1e6, 1) == g["weights_mflop_per_token"]
    assert round((f - 6 * g["n_params"]) / 1e6, 1) == g["attention_mflop_per_token"]
    peak = g["measured_peak_tflops"] * 1e12
    assert int(peak / f) == g["ceiling_tokens_per_s"]
    assert round(100 * oracle.mfu(g["run_tokens_per_s"], f, peak), 1) == g["run_mfu_percent"]
    assert round(100 * oracle.mfu(g["best_tokens_per_s"], f, peak)) == g["best_mfu_percent"]
    assert round(100 * oracle.mfu(g["best_tokens_per_s"], f, g["spec_peak_tflops"] * 1e12)) == \
        g["best_mfu_vs_spec_percent"]


def test_parameter_counts_from_page_listing():
    g = golden("gpt2_shapes.json")
    n_emb = sum(int(np.prod(s)) for s in g["embeddings"].values())
    n_layer = sum(int(np.prod(s)) for s in g["per_layer"].values())
    n_fin = sum(int(np.prod(s)) for s in g["final"].values())
    total = n_emb + g["n_layer"] * n_layer + n_fin
    assert total == 124_439_808
    gpt2_unpadded = M.Config(50257, 1024, 12, 12, 768, 3072)
    assert M.n_params(gpt2_unpadded) == total
    assert M.n_params(GPT2) == 124_475_904
    assert M.n_params(C0) == 108_416
    # the page's Conv1D listing stores c_attn as [in, out]; ours is [out, in]
    specs = dict(M.param_specs(gpt2_unpadded))
    for short, shape in g["per_layer"].items():
        ours = specs["transformer.h.0." + short]
        assert tuple(ours) == tuple(shape[::-1])
    assert round(50257 * 768 / 1e6) - 1 == g["tying_saves_about_millions"] or \
        int(50257 * 768 / 1e6) == g["tying_saves_about_millions"]
    assert g["padded_vocab"] % 32 == 0 and g["padded_vocab"] // 32 == g["padded_vocab_over_32"]
    assert round(50257 / 32, 2) == g["unpadded_vocab_over_32"]


def test_step_arithmetic():
    g = golden("step_arithmetic.json")
    assert g["total_batch_size"] // (g["B"] * g["T"]) == g["grad_accum_steps"]
    assert g["total_batch_size"] // g["T"] == g["sequences_per_step"]
    assert g["total_batch_size"] // (g["B"] * g["T"] * g["ddp_world_size"]) == g["grad_accum_steps_8gpu"]
    assert int(g["total_tokens"] / g["total_batch_size"]) == g["max_steps"]
    assert g["total_batch_size"] == 2 ** 19


# ----------------------------------------------------------------------------
# init generator
# ----------------------------------------------------------------------------

def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        out = I.philox4x32_10(*[np.array([c], dtype=np.uint64) for c in w[:4]], w[4], w[5])
        assert [int(o[0]) for o in out] == w[6:]


def test_init_statistics():
    cfg = M.Config(vocab_size=4096, block_size=256, n_layer=4, n_head=4, n_embd=256, mlp_hidden=1024)
    p = I.init_params(cfg, seed=42)
    for name, shape in M.param_specs(cfg):
        a = p[name].astype(np.float64)
        if len(shape) >= 2:
            std = 0.02 * (2 * cfg.n_layer) ** -0.5 if name.endswith("c_proj.weight") else 0.02
            assert abs(a.std() / std - 1) < 0.01, name
            assert abs(a.mean()) < 4 * std / math.sqrt(a.size)
        elif "ln_" in name and name.endswith("weight"):
            assert np.all(a == 1)
        else:
            assert np.all(a == 0)
    z = I.normal_from_philox(200_000, 3, 7)
    # moments of a standard normal: mean 0, variance 1, kurtosis 3
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert abs((z ** 4).mean() - 3) < 0.05
    # distinct tensors and distinct seeds give distinct streams
    assert not np.allclose(I.normal_from_philox(64, 3, 7), I.normal_from_philox(64, 4, 7))
    assert not np.allclose(I.normal_from_philox(64, 3, 7), I.normal_from_philox(64, 3, 8))


# ----------------------------------------------------------------------------
# the documented PyTorch routines on the CPU, as library primitives
# ----------------------------------------------------------------------------

def test_against_torch_cpu_autograd_and_optimizer():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    cfg = C0
    params = {k: v.astype(np.float64) for k, v in synthetic.random_params(M.param_specs(cfg), seed=12).items()}
    stream = synthetic.uniform_stream(4 * 64 + 1, cfg.vocab_size, seed=13)
    x, y = synthetic.micro_batch(stream, 0, 4, 64)
    y = y.copy()
    y[0, :3] = -1
    scale = 0.5
    loss, _, g = M.fwd_bwd(cfg, params, x, y, scale=scale)

    tp = {k: torch.tensor(v, requires_grad=True) for k, v in params.items()}
    X = torch.tensor(x, dtype=torch.long)
    Y = torch.tensor(y, dtype=torch.long)
    B, T = x.shape
    C, H = cfg.n_embd, cfg.n_head
    h = tp["transformer.wte.weight"][X] + tp["transformer.wpe.weight"][torch.arange(T)]
    for layer in range(cfg.n_layer):
        p = f"transformer.h.{layer}."
        a = F.layer_norm(h, (C,), tp[p + "ln_1.weight"], tp[p + "ln_1.bias"], eps=1e-5)
        qkv = F.linear(a, tp[p + "attn.c_attn.weight"], tp[p + "attn.c_attn.bias"])
        q, k, v = qkv.split(C, dim=2)
        q, k, v = (t.view(B, T, H, C // H).transpose(1, 2) for t in (q, k, v))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.transpose(1, 2).contiguous().view(B, T, C)
        h = h + F.linear(o, tp[p + "attn.c_proj.weight"], tp[p + "attn.c_proj.bias"])
        a = F.layer_norm(h, (C,), tp[p + "ln_2.weight"], tp[p + "ln_2.bias"], eps=1e-5)
        u = F.gelu(F.linear(a, tp[p + "mlp.c_fc.weight"], tp[p + "mlp.c_fc.bias"]), approximate="tanh")
        h = h + F.linear(u, tp[p + "mlp.c_proj.weight"], tp[p + "mlp.c_proj.bias"])
    z = F.layer_norm(h, (C,), tp["transformer.ln_f.weight"], tp["transformer.ln_f.bias"], eps=1e-5)
    logits = z @ tp["transformer.wte.weight"].T
    tl = F.cross_entropy(logits.view(-1, logits.size(-1)), Y.view(-1), ignore_index=-1)
    (tl * scale).backward()
    assert float(tl) == pytest.approx(loss, rel=1e-12)
    for name in params:
        ref = tp[name].grad.numpy()
        np.testing.assert_allclose(g[name], ref, rtol=1e-8, atol=1e-13, err_msg=name)

    # clip_grad_norm_ + AdamW with decay on dim >= 2 only
    mo = {k: np.zeros_like(v) for k, v in params.items()}
    vo = {k: np.zeros_like(v) for k, v in params.items()}
    po = {k: v.copy() for k, v in params.items()}
    go = {k: v.copy() for k, v in g.items()}
    tparams = {k: torch.tensor(v, requires_grad=True) for k, v in params.items()}
    for k in tparams:
        tparams[k].grad = torch.tensor(g[k])
    decay = [tparams[k] for k in tparams if tparams[k].dim() >= 2]
    nodecay = [tparams[k] for k in tparams if tparams[k].dim() < 2]
    opt = torch.optim.AdamW([{"params": decay, "weight_decay": 0.1}, {"params": nodecay, "weight_decay": 0.0}],
                            lr=1e-3, betas=(0.9, 0.95), eps=1e-8)
    for t in (1, 2):
        if t == 2:
            go = {k: v.copy() for k, v in g.items()}
            for k in tparams:
                tparams[k].grad = torch.tensor(g[k])
        tn = float(torch.nn.utils.clip_grad_norm_(list(tparams.values()), 0.05))
        opt.step()
        n = O.clip_adamw_step(po, go, mo, vo, t, 1e-3, max_norm=0.05)
        assert n == pytest.approx(tn, rel=1e-12)
        for k in po:
            np.testing.assert_allclose(po[k], tparams[k].detach().numpy(), rtol=1e-10, atol=1e-14, err_msg=k)
