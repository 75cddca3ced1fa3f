"""End-to-end parity of the training step on the GPU against the oracle,
through the C-ABI (gpt2_init_params, gpt2_fwd_bwd, gpt2_clip_adamw_step,
gpt2_zero_grad), plus the device error paths.

Bars: float32 mode -- loss rel err <= 1e-4, per-tensor grad rel err <= 1e-3;
bf16 mode -- loss rel err <= 1e-2, per-tensor grad cosine >= 0.999,
post-AdamW param max abs diff <= 1e-3.
"""

import math

import numpy as np
import pytest

from gpu_util import announce, cosine, dev, host, load_params, read_named, rel_l2
from oracle import init as OI
from oracle import model as OM
from oracle import optim as OO
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    import gpt_pretraining_step_amd as g
    assert torch.cuda.is_available()
    g.lib()
    return g


def ocfg(c):
    return OM.Config(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


def run_gpu(g, m, x, y, scale=1.0, want_token_loss=False):
    import torch
    tl = torch.zeros(x.shape, dtype=torch.float32, device="cuda") if want_token_loss else None
    loss = m.fwd_bwd(dev(x.astype(np.int32)), dev(y.astype(np.int32)), loss_scale=scale, token_loss=tl)
    st = m.status()
    return float(host(loss)[0]), (host(tl) if tl is not None else None), st


# ---------------------------------------------------------------- fp32 (tiny)

def test_tiny_fp32_step_parity(g):
    """The tiny character-level GPT in float32: one fwd/bwd + clip + AdamW."""
    cfg = g.TINY_CHAR_FP32
    oc = ocfg(cfg)
    announce("tiny fp32 fwd_bwd + clip_adamw")
    m = g.GPT2(cfg)
    params = synthetic.random_params(OM.param_specs(oc), seed=5)
    load_params(m, params)
    m.zero_grad()
    stream = synthetic.uniform_stream(4 * 64 + 1, 66, seed=1337)
    x, y = synthetic.micro_batch(stream, 0, 4, 64)
    loss, tl, st = run_gpu(g, m, x, y, scale=1.0, want_token_loss=True)
    assert st == 0
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    lref, rl, gref = OM.fwd_bwd(oc, p64, x, y)
    assert abs(loss - lref) / abs(lref) <= 1e-4
    np.testing.assert_allclose(tl.reshape(-1), rl, rtol=1e-4, atol=1e-5)
    grads = read_named(m, m.grads)
    worst = max(rel_l2(grads[n], gref[n]) for n in gref if np.linalg.norm(gref[n]) > 0)
    assert worst <= 1e-3, worst

    # clip + AdamW (lr 1e-3, betas 0.9/0.95, wd 0.1, clip 1.0), from the same grads
    ref_p = {k: v.copy() for k, v in p64.items()}
    mo = {k: np.zeros_like(v) for k, v in p64.items()}
    vo = {k: np.zeros_like(v) for k, v in p64.items()}
    gg = {k: grads[k].astype(np.float64) for k in grads}
    nref = OO.clip_adamw_step(ref_p, gg, mo, vo, 1, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0)
    norm = m.clip_adamw_step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0)
    assert m.status() == 0
    assert abs(float(host(norm)[0]) - nref) <= 1e-5 * nref
    newp = read_named(m, m.params)
    for k in ref_p:
        assert np.abs(newp[k] - ref_p[k]).max() <= 1e-6, k
    assert m.step == 1
    m.close()


def test_tiny_fp32_accumulation_identity(g):
    """4 micro-steps of B=1 with loss/4 give the gradient of one B=4 call
    (equal target counts), on the GPU."""
    cfg = g.TINY_CHAR_FP32
    announce("tiny fp32 accumulation identity")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(OM.param_specs(ocfg(cfg)), seed=6))
    stream = synthetic.uniform_stream(4 * 64 + 1, 66, seed=7)
    x, y = synthetic.micro_batch(stream, 0, 4, 64)
    m.zero_grad()
    losses = []
    for k in range(4):
        l, _, st = run_gpu(g, m, x[k:k + 1].copy(), y[k:k + 1].copy(), scale=0.25)
        losses.append(l)
    acc = read_named(m, m.grads)
    m.zero_grad()
    lu, _, _ = run_gpu(g, m, x, y, scale=1.0)
    one = read_named(m, m.grads)
    assert abs(np.mean(losses) - lu) <= 1e-5 * lu
    for k in one:
        if np.linalg.norm(one[k]) > 0:
            assert rel_l2(acc[k], one[k]) <= 1e-5, k
    m.close()


def test_init_params_matches_oracle_generator(g):
    """gpt2_init_params draws the same Philox4x32-10 / Box-Muller stream as the
    oracle's init; biases 0 and LayerNorm gains 1 exactly."""
    cfg = g.ModelConfig(512, 128, 2, 2, 128, 512, 2, g.PRECISION_BF16)
    oc = ocfg(cfg)
    announce("init_params vs oracle")
    m = g.GPT2(cfg)
    m.init_params(seed=42)
    assert m.status() == 0
    got = read_named(m, m.params)
    ref = OI.init_params(oc, seed=42, dtype=np.float64)
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-6, atol=1e-9, err_msg=k)
    shadow = read_named(m, m.shadow)
    np.testing.assert_allclose(shadow["transformer.wte.weight"], got["transformer.wte.weight"], rtol=1e-2, atol=1e-6)
    assert m.step == 0
    m.close()


# ------------------------------------------------------------------- bf16

SMALL_BF16 = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=2, n_embd=128, mlp_hidden=512)


def _bf16_parity(g, cfg, B, T, seed, announce_as):
    oc = ocfg(cfg)
    announce(announce_as)
    m = g.GPT2(cfg)
    params = synthetic.random_params(OM.param_specs(oc), seed=seed)
    load_params(m, params)
    m.zero_grad()
    stream = synthetic.token_stream(B * T + 1, seed=seed)
    stream = np.where(stream < cfg.vocab_size, stream, stream % cfg.vocab_size).astype(np.int32)
    x, y = synthetic.micro_batch(stream, 0, B, T)
    loss, tl, st = run_gpu(g, m, x, y, scale=0.5, want_token_loss=True)
    assert st == 0
    lref, rl, gref = OM.fwd_bwd(oc, params, x, y, scale=0.5)
    grads = read_named(m, m.grads)
    m.close()
    return loss, tl, lref, rl, grads, gref


def test_small_bf16_step_parity(g):
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=3, precision=g.PRECISION_BF16)
    loss, tl, lref, rl, grads, gref = _bf16_parity(g, cfg, 3, 200, 11, "small bf16 fwd_bwd B=3 T=200")
    assert abs(loss - lref) / abs(lref) <= 1e-2
    assert np.abs(tl.reshape(-1) - rl).max() <= 0.05
    for k in gref:
        if np.linalg.norm(gref[k]) > 0:
            c = cosine(grads[k], gref[k])
            assert c >= 0.999, (k, c)


@pytest.mark.timeout(600)
def test_gpt2_124m_bf16_step_parity_b1(g):
    """GPT-2 124M at its real width, one sequence of 1024 tokens: loss and every
    one of the 148 gradient tensors against the float32 oracle."""
    cfg = g.ModelConfig(50304, 1024, 12, 12, 768, 3072, 1, g.PRECISION_BF16)
    loss, tl, lref, rl, grads, gref = _bf16_parity(g, cfg, 1, 1024, 42, "gpt2-124m bf16 fwd_bwd B=1 T=1024")
    assert abs(loss - lref) / abs(lref) <= 1e-2
    worst = min((cosine(grads[k], gref[k]), k) for k in gref if np.linalg.norm(gref[k]) > 0)
    assert worst[0] >= 0.999, worst


def test_small_bf16_causality_bitwise(g):
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=2, precision=g.PRECISION_BF16)
    oc = ocfg(cfg)
    announce("small bf16 causality")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(OM.param_specs(oc), seed=3))
    rng = np.random.default_rng(0)
    x = rng.integers(0, cfg.vocab_size, size=(2, 256)).astype(np.int32)
    y = rng.integers(0, cfg.vocab_size, size=(2, 256)).astype(np.int32)
    for t in (0, 100, 254):
        x2 = x.copy()
        x2[:, t + 1:] = rng.integers(0, cfg.vocab_size, size=(2, 255 - t))
        _, tl1, _ = run_gpu(g, m, x, y, want_token_loss=True)
        _, tl2, _ = run_gpu(g, m, x2, y, want_token_loss=True)
        assert np.array_equal(tl1[:, :t + 1], tl2[:, :t + 1]), t
        assert not np.array_equal(tl1[:, t + 1:], tl2[:, t + 1:]), t
    m.close()


# ------------------------------------------------ full size (B=16, T=1024)

@pytest.fixture(scope="module")
def full(g):
    cfg = g.GPT2_124M
    m = g.GPT2(cfg)
    m.init_params(seed=42)
    stream = synthetic.token_stream(2 * 16 * 1024 + 1)
    yield cfg, m, stream
    m.close()


@pytest.mark.timeout(600)
def test_full_microstep_sampled_token_losses(g, full):
    """At the benchmarked shape (B=16, T=1024) the per-position losses of two
    sampled sequences match the oracle run on those sequences alone (each
    sequence's forward depends only on itself); the mean is near ln V at init."""
    cfg, m, stream = full
    announce("gpt2-124m full micro-step sampled sequences")
    x, y = synthetic.micro_batch(stream, 0, 16, 1024)
    m.zero_grad()
    loss, tl, st = run_gpu(g, m, x, y, scale=1.0, want_token_loss=True)
    assert st == 0
    assert abs(loss - math.log(50257)) <= 0.3
    assert abs(loss - float(tl.mean())) <= 1e-3 * loss
    params = read_named(m, m.params)
    oc = ocfg(cfg)
    for b in (0, 13):
        _, rl, _ = OM.forward(oc, params, x[b:b + 1], y[b:b + 1])
        assert np.abs(tl[b] - rl).max() <= 0.05, b
        assert abs(tl[b].mean() - rl.mean()) <= 1e-2 * rl.mean()
    grads = read_named(m, m.grads)
    assert all(np.isfinite(v).all() for v in grads.values())


@pytest.mark.timeout(600)
def test_full_accumulation_identity_on_gpu(g, full):
    """B=16 in one call vs two B=8 calls with loss/2: same gradients."""
    cfg, m, stream = full
    announce("gpt2-124m accumulation identity B=16 vs 2x8")
    x, y = synthetic.micro_batch(stream, 1, 16, 1024)
    m.zero_grad()
    l1, _, _ = run_gpu(g, m, x, y, scale=1.0)
    one = read_named(m, m.grads)
    m.zero_grad()
    la, _, _ = run_gpu(g, m, x[:8].copy(), y[:8].copy(), scale=0.5)
    lb, _, _ = run_gpu(g, m, x[8:].copy(), y[8:].copy(), scale=0.5)
    two = read_named(m, m.grads)
    assert abs((la + lb) / 2 - l1) <= 1e-4 * l1
    for k in one:
        if np.linalg.norm(one[k]) > 0:
            assert cosine(two[k], one[k]) >= 0.9999, k


@pytest.mark.timeout(600)
def test_full_embedding_gradients_are_deterministic(g, full):
    """The embedding gradients of a micro-step are bitwise identical when it
    is run again: the Zipf stream repeats ids hundreds of times among the
    16,384 rows, and each wte row sums its token's rows in row order (no
    atomics); with the document mask the restarted positions scatter into
    wpe the same way.  So are the 25 LayerNorms' weight and bias gradients
    (every block of a norm backward leaves its column partials, summed in
    block order)."""
    cfg, m, stream = full
    x, y = synthetic.micro_batch(stream, 0, 16, 1024)
    counts = np.bincount(x.reshape(-1))
    assert counts.max() >= 100  # ids really repeat
    for eot in (None, synthetic.EOT_ID):
        announce(f"gpt2-124m embedding gradient determinism, doc mask {eot}")
        m.set_doc_mask(eot)
        runs = []
        for _ in range(2):
            m.zero_grad()
            run_gpu(g, m, x, y)
            gr = read_named(m, m.grads)
            norms = {k: v.copy() for k, v in gr.items() if ".ln_" in k}
            runs.append((gr["transformer.wte.weight"].copy(), gr["transformer.wpe.weight"].copy(), norms))
        assert np.array_equal(runs[0][0], runs[1][0]), eot
        assert np.array_equal(runs[0][1], runs[1][1]), eot
        assert len(runs[0][2]) == 50
        for k in runs[0][2]:
            assert np.array_equal(runs[0][2][k], runs[1][2][k]), (eot, k)
    m.set_doc_mask(None)
    m.zero_grad()


@pytest.mark.timeout(600)
def test_full_optimizer_step_adamw_parity(g, full):
    """Full optimizer step at the benchmarked shape: grads accumulated over
    micro-steps with loss/G, then clip 1.0 + AdamW (lr 6e-4, betas 0.9/0.95,
    eps 1e-8, wd 0.1 on 2-D only).  The update is checked element by element
    against the oracle's clip + AdamW applied to the same gradients."""
    import torch
    cfg, m, stream = full
    G = 2
    announce("gpt2-124m optimizer step")
    m.zero_grad()
    for k in range(G):
        x, y = synthetic.micro_batch(stream, k, 16, 1024)
        run_gpu(g, m, x, y, scale=1.0 / G)
    p_before = read_named(m, m.params)
    g_before = read_named(m, m.grads)
    m_before = read_named(m, m.adam_m)
    v_before = read_named(m, m.adam_v)
    t0 = m.step
    norm = m.clip_adamw_step(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0)
    assert m.status() == 0
    p_after = read_named(m, m.params)
    ref_p = {k: v.astype(np.float64) for k, v in p_before.items()}
    gg = {k: v.astype(np.float64) for k, v in g_before.items()}
    mo = {k: v.astype(np.float64) for k, v in m_before.items()}
    vo = {k: v.astype(np.float64) for k, v in v_before.items()}
    nref = OO.clip_adamw_step(ref_p, gg, mo, vo, t0 + 1, 6e-4, 0.9, 0.95, 1e-8, 0.1, 1.0)
    assert abs(float(host(norm)[0]) - nref) <= 1e-4 * nref
    worst = max(float(np.abs(p_after[k] - ref_p[k]).max()) for k in ref_p)
    assert worst <= 1e-3
    assert worst <= 1e-5  # same gradients: only float32 rounding separates the two
    sh = read_named(m, m.shadow)
    w = p_after["transformer.h.3.mlp.c_fc.weight"]
    assert np.abs(sh["transformer.h.3.mlp.c_fc.weight"] - w).max() <= 2 ** -8 * np.abs(w).max()
    torch.cuda.synchronize()


# ------------------------------------------------------------- error paths

def test_error_paths(g):
    import torch
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=2, precision=g.PRECISION_BF16)
    announce("error paths")
    m = g.GPT2(cfg)
    m.init_params(1)
    x = np.zeros((2, 16), dtype=np.int32)
    y = np.ones((2, 16), dtype=np.int32)
    # host-checkable: B above max_batch, T above block_size
    with pytest.raises(g.GPT2Error) as e:
        m.fwd_bwd(dev(np.zeros((3, 16), np.int32)), dev(np.zeros((3, 16), np.int32)))
    assert e.value.status == g._ffi.GPT2_ERR_SHAPE
    with pytest.raises(g.GPT2Error):
        m.fwd_bwd(dev(np.zeros((1, 257), np.int32)), dev(np.zeros((1, 257), np.int32)))
    # out-of-range token id: flagged, clamped
    xb = x.copy()
    xb[0, 3] = cfg.vocab_size + 5
    _, _, st = run_gpu(g, m, xb, y)
    assert st == g._ffi.GPT2_ERR_BAD_ID
    assert m.status() == 0  # the flag was cleared
    # out-of-range target
    yb = y.copy()
    yb[1, 2] = -7
    _, _, st = run_gpu(g, m, x, yb)
    assert st == g._ffi.GPT2_ERR_BAD_ID
    # no valid target: NaN loss, no gradient added
    m.zero_grad()
    loss, _, st = run_gpu(g, m, x, np.full_like(y, -1))
    assert math.isnan(loss) and st == g._ffi.GPT2_WARN_NO_TARGETS
    assert float(host(m.grads).__abs__().max()) == 0.0
    # non-finite gradient: update skipped (the step counter too), flag raised
    p0 = host(m.params).copy()
    t0 = m.step
    m.grads[5] = float("inf")
    m.clip_adamw_step(lr=1e-3)
    assert m.status() == g._ffi.GPT2_ERR_NONFINITE
    assert np.array_equal(host(m.params), p0)
    assert m.step == t0
    # a finite step afterwards counts from there and uses t0 + 1 in its
    # bias corrections; set_step moves the counter
    m.grads[5] = 0.0
    m.clip_adamw_step(lr=1e-3)
    assert m.status() == 0 and m.step == t0 + 1
    m.step = 41
    assert m.step == 41
    torch.cuda.synchronize()
    m.close()
