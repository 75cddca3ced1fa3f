"""Pins of the oracle's packed-document path ([zero2front] "Document
boundaries, packing and masking": block-diagonal causal attention over the
documents of a window, position ids restarted at each document).

What pins it, other than itself:
  * a hand-worked row whose mask and positions are written out by hand;
  * an independent formulation of the mask (document ids from a running count
    of EOT tokens) checked by brute force on random rows;
  * the reduction to the plain causal model for rows without an EOT;
  * the defining property: a packed window gives the same per-token losses
    as running each of its documents alone from position 0, and its gradient
    is the sum of theirs (the plain path is pinned by finite differences);
  * for the rotary variant, the page's statement that restarting positions
    changes nothing once the mask keeps documents apart.
"""

import numpy as np
import pytest

from oracle import model as M
from oracle import modern as MM
import synthetic

E = 0  # the end-of-text id in these small vocabularies
TINY = M.Config(vocab_size=13, block_size=24, n_layer=2, n_head=2, n_embd=8, mlp_hidden=16)
TINY_ROT = MM.ModernConfig(vocab_size=13, block_size=24, n_layer=2, n_head=2, n_embd=8, mlp_hidden=12)


def test_packed_mask_hand_example():
    # documents: [5 7] (tail of one cut by the window), [E 3 4], [E], [E 9]
    row = np.array([5, 7, E, 3, 4, E, E, 9])
    mask, pos = M.packed_mask(row, E)
    assert pos.tolist() == [0, 1, 0, 1, 2, 0, 0, 1]
    allowed = [np.flatnonzero(mask[t]).tolist() for t in range(8)]
    assert allowed == [[0], [0, 1], [2], [2, 3], [2, 3, 4], [5], [6], [6, 7]]


def _mask_from_document_ids(row, eot):
    # document id = number of EOTs at or before t; a key is visible when it is
    # not after the query and carries the query's document id
    T = row.shape[0]
    doc = np.cumsum(row == eot)
    mask = np.zeros((T, T), dtype=bool)
    pos = np.zeros(T, dtype=np.int64)
    for t in range(T):
        first = min(s for s in range(T) if doc[s] == doc[t])
        pos[t] = t - first
        for s in range(T):
            mask[t, s] = s <= t and doc[s] == doc[t]
    return mask, pos


@pytest.mark.parametrize("p_eot", [0.0, 0.05, 0.3, 1.0])
def test_packed_mask_brute_force(p_eot):
    rng = np.random.default_rng(7)
    for trial in range(20):
        T = int(rng.integers(1, 40))
        row = np.where(rng.random(T) < p_eot, E, rng.integers(1, 9, size=T))
        mask, pos = M.packed_mask(row, E)
        ref_mask, ref_pos = _mask_from_document_ids(row, E)
        assert np.array_equal(mask, ref_mask)
        assert np.array_equal(pos, ref_pos)
        # invariants: every query sees itself, the visible keys are one run
        # ending at the query, and that run has pos + 1 keys
        assert mask.diagonal().all()
        for t in range(T):
            vis = np.flatnonzero(mask[t])
            assert vis[-1] == t and vis.size == vis[-1] - vis[0] + 1 == pos[t] + 1


def _params(specs, seed=3):
    p = synthetic.random_params(specs, seed=seed, matrix_std=0.3, vector_std=0.2)
    return {k: v.astype(np.float64) for k, v in p.items()}


def test_no_eot_reduces_to_causal():
    params = _params(M.param_specs(TINY))
    rng = np.random.default_rng(1)
    x = rng.integers(1, TINY.vocab_size, size=(2, 20))
    y = rng.integers(0, TINY.vocab_size, size=(2, 20))
    mask, pos = M.packed_mask(x[0], E)
    assert np.array_equal(mask, np.tril(np.ones((20, 20), dtype=bool)))
    assert np.array_equal(pos, np.arange(20))
    l0, r0, g0 = M.fwd_bwd(TINY, params, x, y)
    l1, r1, g1 = M.fwd_bwd(TINY, params, x, y, eot=E)
    assert l0 == l1 and np.array_equal(r0, r1)
    for k in g0:
        np.testing.assert_allclose(g1[k], g0[k], rtol=1e-13, atol=1e-15, err_msg=k)


def _documents(row):
    """[start, end) of each document of a row (a new one at every EOT)."""
    starts = sorted({0} | {t for t in range(len(row)) if row[t] == E})
    return list(zip(starts, starts[1:] + [len(row)]))


def _rows_with_documents(T, B, seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(1, TINY.vocab_size, size=(B, T))
    y = rng.integers(0, TINY.vocab_size, size=(B, T))
    x[0, [0, 5, 6, 13]] = E          # EOT first, two in a row, one mid-row
    x[1, [9, T - 1]] = E              # a cut tail first, an EOT as the last token
    y[1, 3] = -1                      # an ignored target
    return x, y


@pytest.mark.parametrize("arch", ["gpt2", "rotary"])
def test_packed_window_equals_separate_documents(arch):
    """Per-token losses of a packed window equal those of its documents run
    alone (positions from 0), and its gradient is the sum of theirs when every
    run divides by the window's count of valid targets."""
    cfg, mod = (TINY, M) if arch == "gpt2" else (TINY_ROT, MM)
    params = _params(mod.param_specs(cfg))
    T, B = 20, 2
    x, y = _rows_with_documents(T, B, seed=11)
    n_valid = int((y >= 0).sum())
    scale = 0.6
    loss, rows, grads = mod.fwd_bwd(cfg, params, x, y, scale=scale, eot=E)
    rows = rows.reshape(B, T)
    summed = {k: np.zeros_like(v) for k, v in grads.items()}
    pieces = 0
    for b in range(B):
        for s, e in _documents(x[b]):
            l_d, r_d, g_d = mod.fwd_bwd(cfg, params, x[b:b + 1, s:e], y[b:b + 1, s:e], scale=scale, n_valid=n_valid)
            np.testing.assert_allclose(rows[b, s:e], r_d, rtol=1e-12, atol=1e-14)
            for k in summed:
                summed[k] += g_d[k]
            pieces += 1
    assert pieces == 4 + 3
    for k in grads:
        np.testing.assert_allclose(grads[k], summed[k], rtol=1e-10, atol=1e-13, err_msg=k)
    # and the packed loss differs from the unmasked one (the mask does something)
    assert abs(mod.fwd_bwd(cfg, params, x, y)[0] - loss) > 1e-6


def test_rotary_restart_changes_nothing_under_the_mask():
    params = _params(MM.param_specs(TINY_ROT))
    x, y = _rows_with_documents(20, 2, seed=12)
    l0, r0, g0 = MM.fwd_bwd(TINY_ROT, params, x, y, eot=E, restart=True)
    l1, r1, g1 = MM.fwd_bwd(TINY_ROT, params, x, y, eot=E, restart=False)
    np.testing.assert_allclose(r1, r0, rtol=1e-12, atol=1e-14)
    for k in g0:
        np.testing.assert_allclose(g1[k], g0[k], rtol=1e-10, atol=1e-13, err_msg=k)


def test_gpt2_restart_matters():
    # with learned positions the restart changes the result: the same window
    # with the mask but positions 0..T-1 is a different function
    params = _params(M.param_specs(TINY))
    x, y = _rows_with_documents(20, 2, seed=13)
    masks, pos = M.packed_rows(x, E)
    assert (pos != np.arange(20)[None]).any()
    l_packed = M.forward(TINY, params, x, y, eot=E)[0]
    l_plain = M.forward(TINY, params, x, y)[0]
    assert abs(l_packed - l_plain) > 1e-6


def test_packed_wpe_gradient_lands_on_restarted_positions():
    # a position no token of the window reaches gets no gradient; wpe row 0
    # gets one from every document start
    params = _params(M.param_specs(TINY))
    x, y = _rows_with_documents(20, 2, seed=14)
    _, pos = M.packed_rows(x, E)
    _, _, g = M.fwd_bwd(TINY, params, x, y, eot=E)
    gw = g["transformer.wpe.weight"]
    reached = set(pos.reshape(-1).tolist())
    for p in range(TINY.block_size):
        assert (np.abs(gw[p]).max() > 0) == (p in reached), p
