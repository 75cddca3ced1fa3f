"""Pins of the oracle learning-rate schedule and loop (CPU only), and the
library's schedule against it.

The schedule [repro-124M] trains with (warmup 300, max_lr 1.5e-3, min_lr 0.1
max_lr, 19,073 steps, cosine decay) is pinned by facts that hold for any
correct warmed-up half-cosine, independent of how the formula is typed: the
linear warmup's values, max_lr at the end of warmup, min_lr at the end, the
mean of max and min halfway through the decay, the decay's symmetry about
that point and its monotonicity, and the average rate over the decay
(the mean of a half cosine is zero).
"""

import math

import numpy as np
import pytest

import oracle as OM

MAX, MIN, WARM, STEPS = 1.5e-3, 1.5e-4, 300, 19073


def test_warmup_is_linear_and_reaches_max():
    assert OM.lr_at(0, MAX, MIN, WARM, STEPS) == pytest.approx(MAX / WARM, rel=1e-12)
    assert OM.lr_at(WARM - 1, MAX, MIN, WARM, STEPS) == pytest.approx(MAX, rel=1e-12)
    d = [OM.lr_at(s + 1, MAX, MIN, WARM, STEPS) - OM.lr_at(s, MAX, MIN, WARM, STEPS) for s in range(WARM - 1)]
    assert np.allclose(d, MAX / WARM, rtol=1e-9)


def test_decay_endpoints_midpoint_and_symmetry():
    assert OM.lr_at(WARM, MAX, MIN, WARM, STEPS) == pytest.approx(MAX, rel=1e-12)
    assert OM.lr_at(STEPS, MAX, MIN, WARM, STEPS) == pytest.approx(MIN, rel=1e-12)
    assert OM.lr_at(STEPS + 500, MAX, MIN, WARM, STEPS) == MIN
    # an even decay length puts a step exactly halfway
    warm, steps = 100, 1100
    mid = (warm + steps) // 2
    assert OM.lr_at(mid, MAX, MIN, warm, steps) == pytest.approx((MAX + MIN) / 2, rel=1e-12)
    for k in (1, 37, 250, 499):
        a = OM.lr_at(mid - k, MAX, MIN, warm, steps) - (MAX + MIN) / 2
        b = OM.lr_at(mid + k, MAX, MIN, warm, steps) - (MAX + MIN) / 2
        assert a == pytest.approx(-b, rel=1e-9)


def test_decay_is_monotone_and_averages_to_the_midpoint():
    lrs = np.array([OM.lr_at(s, MAX, MIN, WARM, STEPS) for s in range(WARM, STEPS + 1)])
    assert np.all(np.diff(lrs) <= 0)
    # trapezoid mean of a half cosine from max to min is their mean
    mean = (lrs[:-1] + lrs[1:]).sum() / 2 / (len(lrs) - 1)
    assert mean == pytest.approx((MAX + MIN) / 2, rel=1e-6)


def test_library_schedule_matches_the_oracle():
    """gpt2_lr_at is a host function of the library: no device needed."""
    from gpt_pretraining_step_amd import _ffi
    L = _ffi.lib()
    for warm, steps in [(WARM, STEPS), (5, 40), (1, 2)]:
        for s in list(range(0, 60)) + [warm - 1, warm, steps - 1, steps, steps + 1, (warm + steps) // 2]:
            if s < 0:
                continue
            got = L.gpt2_lr_at(s, MAX, MIN, warm, steps)
            assert got == pytest.approx(OM.lr_at(s, MAX, MIN, warm, steps), rel=1e-12, abs=0.0), (warm, steps, s)
    assert math.isnan(L.gpt2_lr_at(0, MAX, MIN, 0, STEPS))  # no warmup length: rejected as NaN
    assert math.isnan(L.gpt2_lr_at(0, MAX, MIN, 10, 10))    # no decay phase


def test_oracle_loop_on_a_tiny_model_lowers_the_loss():
    """The oracle loop itself: a 2-layer model overfits one fixed batch (the
    training loop's own smoke test, [zero2front] "train it")."""
    cfg = OM.Config(vocab_size=32, block_size=16, n_layer=2, n_head=2, n_embd=32, mlp_hidden=128)
    params = OM.init_params(cfg, seed=3, dtype=np.float64)
    rng = np.random.default_rng(0)
    tok = rng.integers(0, 32, size=(2, 16)).astype(np.int64)
    tgt = np.roll(tok, -1, axis=1)
    hist = OM.train(cfg, params, lambda s: [(tok, tgt)], 40, OM.fwd_bwd, 3e-3, 3e-4, 5, 40, weight_decay=0.0)
    assert hist[0][0] == pytest.approx(math.log(32), abs=0.1)
    assert hist[-1][0] < 0.5 * hist[0][0]
    assert [h[2] for h in hist[:5]] == pytest.approx([3e-3 * (s + 1) / 5 for s in range(5)])


def _tiny_problem(seed):
    cfg = OM.Config(vocab_size=24, block_size=8, n_layer=2, n_head=2, n_embd=16, mlp_hidden=32)
    params = OM.init_params(cfg, seed=seed, dtype=np.float64)
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, 24, size=(4, 8)).astype(np.int64)
    tgt = rng.integers(0, 24, size=(4, 8)).astype(np.int64)
    return cfg, params, tok, tgt


def test_oracle_loop_micro_batches_equal_their_union():
    """One optimizer step over G = 2 micro-batches with loss / G is the step
    over their union when both hold the same number of targets ([grad-accum]
    "Gradient accumulation averages across micro-steps"; [train-124M] 8.1):
    same parameters, same reported loss and pre-clip norm.  A loop that
    forgot the 1 / G scale would double the gradient (and the norm)."""
    cfg, p0, tok, tgt = _tiny_problem(11)
    pa = {k: v.copy() for k, v in p0.items()}
    pb = {k: v.copy() for k, v in p0.items()}
    halves = [(tok[:2], tgt[:2]), (tok[2:], tgt[2:])]
    ha = OM.train(cfg, pa, lambda s: halves, 1, OM.fwd_bwd, 1e-2, 1e-3, 1, 10, max_norm=1e9)
    hb = OM.train(cfg, pb, lambda s: [(tok, tgt)], 1, OM.fwd_bwd, 1e-2, 1e-3, 1, 10, max_norm=1e9)
    assert ha[0][0] == pytest.approx(hb[0][0], rel=1e-12)
    assert ha[0][1] == pytest.approx(hb[0][1], rel=1e-10)
    for k in p0:
        np.testing.assert_allclose(pa[k], pb[k], rtol=0, atol=1e-12, err_msg=k)
    # the norm is the one of the union's mean-loss gradient, computed directly
    _, _, g = OM.fwd_bwd(cfg, {k: v.copy() for k, v in p0.items()}, tok, tgt)
    assert ha[0][1] == pytest.approx(OM.global_grad_norm(g), rel=1e-10)
    # with the clip active the two runs still agree
    pc = {k: v.copy() for k, v in p0.items()}
    pd = {k: v.copy() for k, v in p0.items()}
    OM.train(cfg, pc, lambda s: halves, 1, OM.fwd_bwd, 1e-2, 1e-3, 1, 10, max_norm=1e-3)
    OM.train(cfg, pd, lambda s: [(tok, tgt)], 1, OM.fwd_bwd, 1e-2, 1e-3, 1, 10, max_norm=1e-3)
    for k in p0:
        np.testing.assert_allclose(pc[k], pd[k], rtol=0, atol=1e-12, err_msg=k)


def test_oracle_loop_two_steps_compose_from_single_steps():
    """Each optimizer step starts from zero gradients ([train-124M] 8.1,
    optimizer.zero_grad() at the top of the step).  With betas 0 (AdamW then
    keeps no history: m = g, v = g^2, bias corrections 1) and a constant
    rate, a two-step run must equal two one-step runs applied in turn; a loop
    that did not zero the gradients would feed step 1's gradient into step 2."""
    cfg, p0, tok, tgt = _tiny_problem(12)
    b0 = [(tok[:2], tgt[:2]), (tok[2:], tgt[2:])]
    b1 = [(tok[[1, 3]], tgt[[0, 2]]), (tok[[0, 2]], tgt[[1, 3]])]
    hp = dict(beta1=0.0, beta2=0.0, max_norm=0.5)
    pa = {k: v.copy() for k, v in p0.items()}
    ha = OM.train(cfg, pa, lambda s: b0 if s == 0 else b1, 2, OM.fwd_bwd, 5e-3, 5e-3, 1, 10, **hp)
    pb = {k: v.copy() for k, v in p0.items()}
    h0 = OM.train(cfg, pb, lambda s: b0, 1, OM.fwd_bwd, 5e-3, 5e-3, 1, 10, **hp)
    h1 = OM.train(cfg, pb, lambda s: b1, 1, OM.fwd_bwd, 5e-3, 5e-3, 1, 10, **hp)
    assert [ha[0][0], ha[1][0]] == pytest.approx([h0[0][0], h1[0][0]], rel=1e-12)
    assert [ha[0][1], ha[1][1]] == pytest.approx([h0[0][1], h1[0][1]], rel=1e-10)
    for k in p0:
        np.testing.assert_allclose(pa[k], pb[k], rtol=0, atol=1e-12, err_msg=k)
    # and the second step really moved the weights (the pin is not vacuous)
    assert max(float(np.abs(pa[k] - p0[k]).max()) for k in p0) > 1e-3
