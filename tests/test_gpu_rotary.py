"""The rotary variant on the GPU (RMSNorm, RoPE, SwiGLU, no position table, no
biases): its kernels through the single-op C-ABI entry points, and the whole
micro-step against the oracle of the variant.

Bars as for GPT-2 in bf16: loss rel err <= 1e-2, per-tensor grad cosine
>= 0.999; the kernels against the oracle's pieces on the same bf16-rounded
inputs.
"""

import math

import numpy as np
import pytest

from gpu_util import announce, bf16_round, cosine, dev, host, load_params, read_named
from oracle import init as OI
from oracle import modern as MM
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
    return MM.ModernConfig(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


# ------------------------------------------------------------------ pieces

def test_rope_table_vs_oracle(g):
    announce("rope table T=1024")
    tab = host(g.op_rope_table(1024))
    cos, sin = MM.rope_tables(1024, 64)
    np.testing.assert_allclose(tab[:, :, 0], cos[:, :32], rtol=0, atol=2e-7)
    np.testing.assert_allclose(tab[:, :, 1], sin[:, :32], rtol=0, atol=2e-7)


@pytest.mark.parametrize("rows,T,C", [(300, 100, 256), (2048, 1024, 768)])
def test_rope_bwd_vs_oracle(g, rows, T, C):
    """The backward rotation of the q and k blocks of a [rows, 3C] gradient,
    in place; the v block is left alone."""
    import torch
    announce(f"rope bwd rows={rows} T={T} C={C}")
    rng = np.random.default_rng(rows)
    d = bf16_round(rng.standard_normal((rows, 3 * C)).astype(np.float32))
    t = dev(d, torch.bfloat16)
    g.op_rope_bwd(t, T, C, g.op_rope_table(T))
    out = host(t)
    cos, sin = MM.rope_tables(T, 64)
    pos = np.arange(rows) % T
    H = C // 64
    for blk in (0, 1):
        z = d[:, blk * C:(blk + 1) * C].reshape(rows, H, 64).astype(np.float64)
        ref = MM.rope_bwd(z, cos[pos][:, None, :], sin[pos][:, None, :]).reshape(rows, C)
        np.testing.assert_allclose(out[:, blk * C:(blk + 1) * C], ref, rtol=1e-2, atol=1e-2)
    assert np.array_equal(out[:, 2 * C:], d[:, 2 * C:])


@pytest.mark.parametrize("B,T,H,Hkv", [(2, 300, 4, 4), (1, 1024, 6, 2)])
def test_attention_bwd_fused_rope(g, B, T, H, Hkv):
    """gpt2_op_attention_bwd with the rotary table rotates dq and dk back in
    registers: against the oracle (attention backward, then the transpose of
    the rotation, in float64) and against the two-pass path (backward, then
    gpt2_op_rope_bwd); dv is untouched."""
    import torch
    from oracle import model as OM
    hd = 64
    announce(f"attention bwd + fused rope B={B} T={T} H={H} Hkv={Hkv}")
    rng = np.random.default_rng(T + H)
    C, Ckv = H * hd, Hkv * hd
    W = C + 2 * Ckv
    qkv = bf16_round(rng.standard_normal((B * T, W)).astype(np.float32))
    dy = bf16_round(rng.standard_normal((B * T, C)).astype(np.float32))
    dq_ = dev(qkv, torch.bfloat16)
    y = torch.zeros((B * T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dq_, y, lse, B, T, H, hd, n_kv_head=Hkv)
    tab = g.op_rope_table(T)
    fused = torch.zeros((B * T, W), dtype=torch.bfloat16, device="cuda")
    g.op_attention_bwd(dq_, y, dev(dy, torch.bfloat16), lse, fused, B, T, H, hd, n_kv_head=Hkv, rope=tab)
    two = torch.zeros((B * T, W), dtype=torch.bfloat16, device="cuda")
    g.op_attention_bwd(dq_, y, dev(dy, torch.bfloat16), lse, two, B, T, H, hd, n_kv_head=Hkv)
    # the separate pass rotates the first `C + Ckv` columns (q and k heads)
    assert g.lib().gpt2_op_rope_bwd(None, two.data_ptr(), B * T, W, C + Ckv, T, tab.data_ptr()) == 0
    f, t2 = host(fused), host(two)
    assert np.array_equal(f[:, C + Ckv:], t2[:, C + Ckv:])  # dv: no rotation, same kernel
    np.testing.assert_allclose(f[:, :C + Ckv], t2[:, :C + Ckv], rtol=2e-2, atol=2e-2)
    # oracle: per-head attention backward on the shared heads, then the
    # transpose of the rotation at each row's position
    cos, sin = MM.rope_tables(T, 64)
    x = qkv.reshape(B, T, W).astype(np.float64)
    ref = np.zeros((B, T, W))
    grp = H // Hkv
    yh = host(y).reshape(B, T, C).astype(np.float64)
    for b in range(B):
        for h in range(H):
            j = h // grp
            q, k = x[b, :, h * hd:(h + 1) * hd], x[b, :, C + j * hd:C + (j + 1) * hd]
            v = x[b, :, C + Ckv + j * hd:C + Ckv + (j + 1) * hd]
            _, p = OM.attention_fwd(q, k, v)
            dq, dk, dv = OM.attention_bwd(dy.reshape(B, T, C)[b, :, h * hd:(h + 1) * hd].astype(np.float64), q, k, v, p)
            ref[b, :, h * hd:(h + 1) * hd] = MM.rope_bwd(dq, cos, sin)
            ref[b, :, C + j * hd:C + (j + 1) * hd] += MM.rope_bwd(dk, cos, sin)
            ref[b, :, C + Ckv + j * hd:C + Ckv + (j + 1) * hd] += dv
    ref = ref.reshape(B * T, W)
    for name, sl in (("dq", slice(0, C)), ("dk", slice(C, C + Ckv))):
        assert cosine(f[:, sl], ref[:, sl]) > 0.999, name
        assert np.abs(f[:, sl] - ref[:, sl]).max() <= 3e-2 * max(1.0, np.abs(ref[:, sl]).max()), name
    # a misaligned or float32 table is refused
    with pytest.raises(g.GPT2Error):
        g.op_attention_bwd(dq_, y, dev(dy, torch.bfloat16), lse, fused, B, T, H, hd, n_kv_head=Hkv,
                           rope=tab.view(-1)[2:])


@pytest.mark.parametrize("rows,C,dyb", [(1, 256, False), (1000, 768, True), (129, 1024, False), (70, 512, True)])
def test_rmsnorm_vs_oracle(g, rows, C, dyb):
    import torch
    announce(f"rmsnorm rows={rows} C={C} dy_bf16={dyb}")
    rng = np.random.default_rng(rows + C)
    x = (rng.standard_normal((rows, C)) * 2 + 0.3).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    y_ref, cache = MM.rmsnorm_fwd(x.astype(np.float64), w.astype(np.float64))
    y = torch.zeros((rows, C), dtype=torch.bfloat16, device="cuda")
    rstd = torch.zeros(rows, dtype=torch.float32, device="cuda")
    xd = dev(x)
    g.op_rmsnorm_fwd(xd, dev(w), y, rstd)
    np.testing.assert_allclose(host(y), y_ref, rtol=1e-2, atol=1e-2)
    np.testing.assert_allclose(host(rstd), cache[1][:, 0], rtol=1e-5)
    dy = rng.standard_normal((rows, C)).astype(np.float32)
    if dyb:
        dy = synthetic.round_to_bf16(dy)
    dx0 = rng.standard_normal((rows, C)).astype(np.float32)
    dxr, dwr = MM.rmsnorm_bwd(dy.astype(np.float64), cache, w.astype(np.float64))
    dx = dev(dx0)
    dxb = torch.zeros((rows, C), dtype=torch.bfloat16, device="cuda")
    dw = dev(np.ones(C, dtype=np.float32))
    g.op_rmsnorm_bwd(dev(dy, torch.bfloat16) if dyb else dev(dy), xd, rstd, dev(w), dx, dw, dx_bf16=dxb)
    np.testing.assert_allclose(host(dx), dx0 + dxr, rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(host(dw), 1 + dwr, rtol=1e-4, atol=1e-3)
    assert torch.equal(dxb, dx.to(torch.bfloat16))


@pytest.mark.parametrize("M,C,K,T", [(520, 256, 200, 100), (1024, 768, 768, 1024)])
def test_gemm_rope_epilogue(g, M, C, K, T):
    """qkv = a W^T with q and k rotated in the epilogue (rows at positions
    m % T); v unrotated.  Ragged M takes the checked edge tiles."""
    import torch
    announce(f"gemm ROPE M={M} C={C} K={K} T={T}")
    rng = np.random.default_rng(M + K)
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    W = bf16_round((rng.standard_normal((3 * C, K)) * 0.1).astype(np.float32))
    P = A.astype(np.float64) @ W.astype(np.float64).T
    cos, sin = MM.rope_tables(T, 64)
    pos = np.arange(M) % T
    H = C // 64
    ref = P.copy()
    for blk in (0, 1):
        z = P[:, blk * C:(blk + 1) * C].reshape(M, H, 64)
        ref[:, blk * C:(blk + 1) * C] = MM.rope_fwd(z, cos[pos][:, None, :], sin[pos][:, None, :]).reshape(M, C)
    out = torch.zeros((M, 3 * C), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dev(A, torch.bfloat16), dev(W, torch.bfloat16), out, M, 3 * C, K, epilogue=g.EPI_ROPE,
              rope=g.op_rope_table(T), rope_period=T, rope_cols=2 * C)
    np.testing.assert_allclose(host(out), ref, rtol=1e-2, atol=2e-2)


@pytest.mark.parametrize("M,F,K", [(520, 160, 128), (2048, 2048, 768)])
def test_gemm_swiglu_epilogue(g, M, F, K):
    """[gate | up] = a [W_gate; W_up]^T; act = silu(gate) up from the bf16
    gate and up; F = 160 leaves a partly filled column tile."""
    import torch
    announce(f"gemm SWIGLU M={M} F={F} K={K}")
    rng = np.random.default_rng(M + F)
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    W = bf16_round((rng.standard_normal((2 * F, K)) * 0.1).astype(np.float32))
    P = A.astype(np.float64) @ W.astype(np.float64).T
    act = torch.zeros((M, F), dtype=torch.bfloat16, device="cuda")
    gu = torch.zeros((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dev(A, torch.bfloat16), dev(W, torch.bfloat16), act, M, 2 * F, K, epilogue=g.EPI_SWIGLU, C2=gu)
    gu_h = host(gu)
    np.testing.assert_allclose(gu_h, P, rtol=1e-2, atol=1e-2)
    gate, up = gu_h[:, :F].astype(np.float64), gu_h[:, F:].astype(np.float64)
    np.testing.assert_allclose(host(act), MM.silu(gate) * up, rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("M,F,K", [(520, 160, 200), (2048, 2048, 768)])
def test_gemm_swiglu_bwd_epilogue(g, M, F, K):
    """d(act) = dR W_down, then dgate = d(act) up silu'(gate) and
    dup = d(act) silu(gate), written side by side."""
    import torch
    announce(f"gemm SWIGLU_BWD M={M} F={F} K={K}")
    rng = np.random.default_rng(M + 3 * F)
    dR = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    Wd = bf16_round((rng.standard_normal((K, F)) * 0.1).astype(np.float32))   # [C, F]: K-slow operand
    GU = bf16_round((rng.standard_normal((M, 2 * F)) * 2).astype(np.float32))
    dact = dR.astype(np.float64) @ Wd.astype(np.float64)
    gate, up = GU[:, :F].astype(np.float64), GU[:, F:].astype(np.float64)
    out = torch.zeros((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dev(dR, torch.bfloat16), dev(Wd, torch.bfloat16), out, M, F, K, a_kmajor=True, b_kmajor=False,
              epilogue=g.EPI_SWIGLU_BWD, U=dev(GU, torch.bfloat16))
    o = host(out)
    np.testing.assert_allclose(o[:, :F], dact * up * MM.silu_grad(gate), rtol=2e-2, atol=2e-2)
    np.testing.assert_allclose(o[:, F:], dact * MM.silu(gate), rtol=2e-2, atol=2e-2)


def test_rotary_epilogues_reject_bad_arguments(g):
    import torch
    announce("rotary epilogue argument checks")
    A = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((192, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((64, 192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GPT2Error):  # rotated columns without a table
        g.op_gemm(A, W, out, 64, 192, 64, epilogue=g.EPI_ROPE, rope_period=64, rope_cols=128)
    with pytest.raises(g.GPT2Error):  # SwiGLU needs K % 64 == 0 and C2
        g.op_gemm(A[:, :40].contiguous(), W[:128, :40].contiguous(), out[:, :64].contiguous(), 64, 128, 40,
                  epilogue=g.EPI_SWIGLU, C2=out[:, :128].contiguous())
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, W[:128].contiguous(), out[:, :64].contiguous(), 64, 128, 64, epilogue=g.EPI_SWIGLU)
    with pytest.raises(g.GPT2Error):  # float32 output
        g.op_gemm(A, W, torch.zeros((64, 192), device="cuda"), 64, 192, 64, epilogue=g.EPI_ROPE,
                  rope=g.op_rope_table(64), rope_period=64, rope_cols=128)


# ------------------------------------------------------------ whole model

SMALL = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=4, n_embd=256, mlp_hidden=160)


def _parity(g, cfg, B, T, seed, what):
    oc = ocfg(cfg)
    announce(what)
    m = g.GPT2(cfg)
    params = synthetic.random_params(MM.param_specs(oc), seed=seed)
    load_params(m, params)
    m.zero_grad()
    stream = synthetic.token_stream(B * T + 1, seed=seed)
    stream = np.where(stream < cfg.vocab_size, stream, stream % cfg.vocab_size).astype(np.int32)
    x, y = synthetic.micro_batch(stream, 0, B, T)
    import torch
    tl = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    loss = m.fwd_bwd(dev(x), dev(y), loss_scale=0.5, token_loss=tl)
    assert m.status() == 0
    lref, rl, gref = MM.fwd_bwd(oc, params, x, y, scale=0.5)
    grads = read_named(m, m.grads)
    m.close()
    return float(host(loss)[0]), host(tl), lref, rl, grads, gref


def test_rotary_small_step_parity(g):
    cfg = g.ModelConfig(**SMALL, max_batch=3, precision=g.PRECISION_BF16, arch=g.ARCH_ROTARY)
    loss, tl, lref, rl, grads, gref = _parity(g, cfg, 3, 200, 11, "rotary small fwd_bwd B=3 T=200")
    assert abs(loss - lref) / abs(lref) <= 1e-2
    assert np.abs(tl.reshape(-1) - rl).max() <= 0.05
    for k in gref:
        if np.linalg.norm(gref[k]) > 0:
            c = cosine(grads[k], gref[k])
            assert c >= 0.999, (k, c)


def test_rotary_norm_gradients_are_reproducible(g):
    """The RMSNorm weight gradients (5 norms, no bias) come from per-block
    column partials summed in block order: a rerun of the same micro-step
    gives the same bits."""
    import torch
    cfg = g.ModelConfig(**SMALL, max_batch=3, precision=g.PRECISION_BF16, arch=g.ARCH_ROTARY)
    announce("rotary norm gradient reproducibility B=3 T=256")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(MM.param_specs(ocfg(cfg)), seed=5))
    rng = np.random.default_rng(1)
    x = rng.integers(0, cfg.vocab_size, size=(3, 256)).astype(np.int32)
    y = rng.integers(0, cfg.vocab_size, size=(3, 256)).astype(np.int32)
    runs = []
    for _ in range(2):
        m.zero_grad()
        m.fwd_bwd(dev(x), dev(y), loss_scale=1.0)
        torch.cuda.synchronize()
        gr = read_named(m, m.grads)
        runs.append({k: v.copy() for k, v in gr.items() if "norm" in k or ".ln_" in k})
    assert len(runs[0]) == 2 * cfg.n_layer + 1, sorted(runs[0])
    for k in runs[0]:
        assert np.array_equal(runs[0][k], runs[1][k]), k
    m.close()


@pytest.mark.timeout(600)
def test_rotary_124m_step_parity_b1(g):
    """The variant at its real width, one sequence of 1024 tokens: loss and
    every gradient tensor against the float32 oracle."""
    cfg = g.ModelConfig(50304, 1024, 12, 12, 768, 2048, 1, g.PRECISION_BF16, g.ARCH_ROTARY)
    loss, tl, lref, rl, grads, gref = _parity(g, cfg, 1, 1024, 42, "rotary 124m fwd_bwd B=1 T=1024")
    assert abs(loss - lref) / abs(lref) <= 1e-2
    worst = min((cosine(grads[k], gref[k]), k) for k in gref if np.linalg.norm(gref[k]) > 0)
    assert worst[0] >= 0.999, worst


def test_rotary_causality_bitwise(g):
    import torch
    cfg = g.ModelConfig(**SMALL, max_batch=2, precision=g.PRECISION_BF16, arch=g.ARCH_ROTARY)
    announce("rotary causality")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(MM.param_specs(ocfg(cfg)), seed=3))
    rng = np.random.default_rng(0)
    x = rng.integers(0, cfg.vocab_size, size=(2, 256)).astype(np.int32)
    y = rng.integers(0, cfg.vocab_size, size=(2, 256)).astype(np.int32)
    for t in (0, 100, 254):
        x2 = x.copy()
        x2[:, t + 1:] = rng.integers(0, cfg.vocab_size, size=(2, 255 - t))
        outs = []
        for xx in (x, x2):
            tl = torch.zeros(xx.shape, dtype=torch.float32, device="cuda")
            m.fwd_bwd(dev(xx), dev(y), loss_scale=1.0, token_loss=tl)
            outs.append(host(tl))
        assert np.array_equal(outs[0][:, :t + 1], outs[1][:, :t + 1]), t
        assert not np.array_equal(outs[0][:, t + 1:], outs[1][:, t + 1:]), t
    m.close()


def test_rotary_init_params_matches_oracle_generator(g):
    """Same Philox4x32-10 / Box-Muller stream as GPT-2 (tensor k = position in
    the variant's table order); std 0.02, residual projections 0.02/sqrt(2L),
    RMSNorm weights 1."""
    cfg = g.ModelConfig(**SMALL, max_batch=1, precision=g.PRECISION_BF16, arch=g.ARCH_ROTARY)
    oc = ocfg(cfg)
    announce("rotary init_params")
    m = g.GPT2(cfg)
    m.init_params(seed=42)
    assert m.status() == 0
    got = read_named(m, m.params)
    for k, (name, shape) in enumerate(MM.param_specs(oc)):
        if len(shape) == 1:
            assert np.array_equal(got[name], np.ones(shape, dtype=np.float32)), name
            continue
        n = int(np.prod(shape))
        ref = (MM.init_std(oc, name, shape) * OI.normal_from_philox(n, k, 42)).reshape(shape)
        np.testing.assert_allclose(got[name], ref, rtol=1e-6, atol=1e-9, err_msg=name)
    m.close()


@pytest.mark.timeout(600)
def test_rotary_full_microstep_sampled_token_losses(g):
    """At the variant's benchmarked shape (B=64, T=1024) the per-position
    losses of two sampled sequences match the oracle run on those sequences
    alone; the mean loss is near ln V at init; gradients are finite."""
    cfg = g.GPT2_ROTARY_124M
    announce("rotary 124m full micro-step B=64 sampled sequences")
    m = g.GPT2(cfg)
    m.init_params(seed=42)
    stream = synthetic.token_stream(64 * 1024 + 1)
    x, y = synthetic.micro_batch(stream, 0, 64, 1024)
    import torch
    tl = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    m.zero_grad()
    loss = float(host(m.fwd_bwd(dev(x), dev(y), loss_scale=1.0, token_loss=tl))[0])
    assert m.status() == 0
    tl = host(tl)
    assert abs(loss - math.log(50257)) <= 0.3
    assert abs(loss - float(tl.mean())) <= 1e-3 * loss
    params = read_named(m, m.params)
    oc = ocfg(cfg)
    for b in (0, 41):
        _, rl, _ = MM.forward(oc, params, x[b:b + 1], y[b:b + 1])
        assert np.abs(tl[b] - rl).max() <= 0.05, b
        assert abs(tl[b].mean() - rl.mean()) <= 1e-2 * rl.mean()
    grads = read_named(m, m.grads)
    assert all(np.isfinite(v).all() for v in grads.values())
    m.close()
