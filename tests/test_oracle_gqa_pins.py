"""Pins of the oracle's grouped-query attention in the rotary variant
([fast-1gpu] "Step 2: the attention kernel": n_head / n_kv_head query heads
share each key/value head, the key and value heads repeated with
repeat_interleave).

What pins it, other than itself:
  * the equivalence that defines it: a grouped-query model equals the
    multi-head model whose k and v projection rows are those of the shared
    head, repeated for every query head of its group (repeat_interleave
    order); the multi-head model's gradient of those repeated rows, summed
    over each group, is the grouped model's gradient (chain rule through the
    repeat), and every other gradient is the same;
  * finite differences on the k and v rows of the grouped model;
  * n_kv_head == n_head is the plain multi-head model.
"""

import numpy as np
import pytest

from oracle import modern as MM
import synthetic

GQA = MM.ModernConfig(vocab_size=17, block_size=12, n_layer=2, n_head=6, n_embd=24, mlp_hidden=20, n_kv_head=2)
MHA = MM.ModernConfig(vocab_size=17, block_size=12, n_layer=2, n_head=6, n_embd=24, mlp_hidden=20)


def _params(cfg, seed=4):
    p = synthetic.random_params(MM.param_specs(cfg), seed=seed, matrix_std=0.3, vector_std=0.2)
    return {k: v.astype(np.float64) for k, v in p.items()}


def _batch(seed=6, B=2, T=10):
    rng = np.random.default_rng(seed)
    return rng.integers(0, GQA.vocab_size, size=(B, T)), rng.integers(0, GQA.vocab_size, size=(B, T))


def _expand(cfg_g, w):
    """c_attn of the grouped model -> c_attn of the equivalent multi-head
    model: q rows kept, k and v head rows repeated over each group."""
    C, hd, Hkv = cfg_g.n_embd, cfg_g.head_dim, cfg_g.kv_heads
    grp = cfg_g.n_head // Hkv
    q, k, v = w[:C], w[C:C + Hkv * hd], w[C + Hkv * hd:]
    rep = lambda m: np.concatenate([m[(j // grp) * hd:(j // grp + 1) * hd] for j in range(cfg_g.n_head)], axis=0)
    return np.concatenate([q, rep(k), rep(v)], axis=0)


def _fold(cfg_g, gm):
    """Gradient of the expanded c_attn -> gradient of the grouped one (sum
    of each group's repeated rows)."""
    C, hd, Hkv = cfg_g.n_embd, cfg_g.head_dim, cfg_g.kv_heads
    grp = cfg_g.n_head // Hkv
    q, k, v = gm[:C], gm[C:2 * C], gm[2 * C:]
    fold = lambda m: np.concatenate(
        [sum(m[j * hd:(j + 1) * hd] for j in range(i * grp, (i + 1) * grp)) for i in range(Hkv)], axis=0)
    return np.concatenate([q, fold(k), fold(v)], axis=0)


def test_shapes():
    specs = dict(MM.param_specs(GQA))
    assert specs["transformer.h.0.attn.c_attn.weight"] == (24 + 2 * 8, 24)
    assert MM.n_params(GQA) < MM.n_params(MHA)


@pytest.mark.parametrize("eot", [None, 3])
def test_grouped_equals_expanded_multi_head(eot):
    pg = _params(GQA)
    pm = dict(pg)
    for layer in range(GQA.n_layer):
        k = f"transformer.h.{layer}.attn.c_attn.weight"
        pm[k] = _expand(GQA, pg[k])
    x, y = _batch()
    if eot is not None:
        x[0, [0, 4]] = eot
        x[1, 7] = eot
    lg, rg, gg = MM.fwd_bwd(GQA, pg, x, y, scale=0.7, eot=eot)
    lm, rm, gm = MM.fwd_bwd(MHA, pm, x, y, scale=0.7, eot=eot)
    assert lg == pytest.approx(lm, rel=1e-13)
    np.testing.assert_allclose(rg, rm, rtol=1e-12, atol=1e-14)
    for k in gg:
        ref = _fold(GQA, gm[k]) if k.endswith("c_attn.weight") else gm[k]
        np.testing.assert_allclose(gg[k], ref, rtol=1e-10, atol=1e-13, err_msg=k)
    # and the grouping matters: pairing query head j with kv head j % n_kv_head
    # (the other plausible order) is a different model
    pw = dict(pm)
    C, hd = GQA.n_embd, GQA.head_dim
    for layer in range(GQA.n_layer):
        k = f"transformer.h.{layer}.attn.c_attn.weight"
        w = pg[k]
        kk, vv = w[C:C + 2 * hd], w[C + 2 * hd:]
        tile = lambda m: np.concatenate([m[(j % 2) * hd:(j % 2 + 1) * hd] for j in range(6)], axis=0)
        pw[k] = np.concatenate([w[:C], tile(kk), tile(vv)], axis=0)
    assert abs(MM.forward(MHA, pw, x, y, eot=eot)[0] - lg) > 1e-6


def test_grouped_finite_differences_on_kv_rows():
    p = _params(GQA, seed=8)
    x, y = _batch(seed=9)
    _, _, g = MM.fwd_bwd(GQA, p, x, y)
    name = "transformer.h.1.attn.c_attn.weight"
    w = p[name]
    rng = np.random.default_rng(3)
    eps = 1e-6
    for _ in range(12):
        r = int(rng.integers(GQA.n_embd, w.shape[0]))  # a k or v row
        c = int(rng.integers(0, w.shape[1]))
        old = w[r, c]
        w[r, c] = old + eps
        lp = MM.forward(GQA, p, x, y)[0]
        w[r, c] = old - eps
        lm = MM.forward(GQA, p, x, y)[0]
        w[r, c] = old
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - g[name][r, c]) <= 1e-6 * max(1.0, abs(fd)), (r, c, fd, g[name][r, c])


def test_kv_heads_equal_heads_is_multi_head():
    cfg = MM.ModernConfig(vocab_size=17, block_size=12, n_layer=2, n_head=6, n_embd=24, mlp_hidden=20, n_kv_head=6)
    p = _params(MHA)
    x, y = _batch()
    a = MM.fwd_bwd(cfg, p, x, y)
    b = MM.fwd_bwd(MHA, p, x, y)
    assert a[0] == b[0]
    for k in a[2]:
        assert np.array_equal(a[2][k], b[2][k]), k
