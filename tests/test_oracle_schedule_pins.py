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
