"""Pins of the modern-variant oracle (RMSNorm, RoPE, SwiGLU, no position table,
no biases) against what the mathematics and the published definitions fix:
finite differences in float64, closed forms of the rotation, invariants of
RMSNorm, the documented PyTorch CPU routines, the parameter count of the
variant and bitwise causality.
"""

import math

import numpy as np
import pytest

from oracle import flops as FL
from oracle import model as M
from oracle import modern as MM
import synthetic

TINY = MM.ModernConfig(vocab_size=11, block_size=8, n_layer=2, n_head=2, n_embd=8, mlp_hidden=12)
FULL = MM.ModernConfig(vocab_size=50304, block_size=1024, n_layer=12, n_head=12, n_embd=768, mlp_hidden=2048)


def tiny_params(seed=3):
    p = synthetic.random_params(MM.param_specs(TINY), seed=seed, matrix_std=0.3, vector_std=0.2)
    return {k: v.astype(np.float64) for k, v in p.items()}


def tiny_batch(seed=5, B=2, T=6, ignore=()):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, TINY.vocab_size, size=(B, T))
    y = rng.integers(0, TINY.vocab_size, size=(B, T))
    for (b, t) in ignore:
        y[b, t] = -1
    return x, y


# ----------------------------------------------------------------------------
# whole model
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("ignore", [(), ((0, 1), (1, 5))])
def test_finite_differences_every_tensor(ignore):
    params = tiny_params()
    x, y = tiny_batch(ignore=ignore)
    scale = 0.7
    _, _, g = MM.fwd_bwd(TINY, params, x, y, scale=scale)
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name, shape in MM.param_specs(TINY):
        flat = params[name].reshape(-1)
        for j in rng.choice(flat.size, size=min(flat.size, 12), replace=False):
            old = flat[j]
            flat[j] = old + eps
            lp = MM.forward(TINY, params, x, y)[0]
            flat[j] = old - eps
            lm = MM.forward(TINY, params, x, y)[0]
            flat[j] = old
            fd = scale * (lp - lm) / (2 * eps)
            an = g[name].reshape(-1)[j]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, j, fd, an)
    # one directional derivative over all tensors at once
    d = {k: np.random.default_rng(7).standard_normal(v.shape) for k, v in params.items()}
    pp = {k: v + eps * d[k] for k, v in params.items()}
    pm = {k: v - eps * d[k] for k, v in params.items()}
    fd = scale * (MM.forward(TINY, pp, x, y)[0] - MM.forward(TINY, pm, x, y)[0]) / (2 * eps)
    an = sum(float((g[k] * d[k]).sum()) for k in params)
    assert fd == pytest.approx(an, rel=1e-7)


def test_causality_bitwise():
    params = {k: v.astype(np.float32) for k, v in tiny_params().items()}
    x, y = tiny_batch(B=1, T=8)
    _, rl0, _ = MM.forward(TINY, params, x, y)
    t = 3
    x2 = x.copy()
    x2[0, t + 1:] = (x2[0, t + 1:] + 1) % TINY.vocab_size
    _, rl1, _ = MM.forward(TINY, params, x2, y)
    assert np.array_equal(rl0[:t + 1], rl1[:t + 1])
    assert not np.array_equal(rl0[t + 1:], rl1[t + 1:])


def test_initial_loss_near_log_vocab():
    """With N(0, 0.02) weights and unit-RMS final states the logits have a
    standard deviation of about 0.02 sqrt(C) = 0.16, so the loss over 32
    random targets is ln V within a few times 0.16 / sqrt(32)."""
    cfg = MM.ModernConfig(vocab_size=512, block_size=16, n_layer=2, n_head=2, n_embd=64, mlp_hidden=96)
    rng = np.random.default_rng(0)
    params = {}
    for name, shape in MM.param_specs(cfg):
        std = MM.init_std(cfg, name, shape)
        params[name] = (np.ones(shape) if len(shape) == 1 else std * rng.standard_normal(shape))
    x = rng.integers(0, cfg.vocab_size, size=(2, 16))
    y = rng.integers(0, cfg.vocab_size, size=(2, 16))
    loss = MM.forward(cfg, params, x, y)[0]
    assert abs(loss - math.log(cfg.vocab_size)) < 0.1


def test_parameter_count_and_flops_of_the_variant():
    """wte 50304x768 + 12 x (2 RMSNorm weights, c_attn 3Cx C, c_proj CxC,
    gate+up 2Fx C, down CxF) + ln_f, no biases, no position table."""
    assert MM.n_params(FULL) == 123_587_328
    assert FL.flops_per_token(FULL, 1024, n=MM.n_params(FULL)) == 854_770_176


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def test_rope_two_dims_is_the_plane_rotation():
    """hd = 2: one pair, frequency 1; rotate_half(x) = (-x1, x0), so x cos +
    rotate_half(x) sin is the rotation of the plane by angle t."""
    cos, sin = MM.rope_tables(5, 2)
    x = np.array([[0.3, -1.2]] * 5)
    out = MM.rope_fwd(x, cos, sin)
    for t in range(5):
        c, s = math.cos(t), math.sin(t)
        assert out[t, 0] == pytest.approx(0.3 * c + 1.2 * s, abs=1e-15)
        assert out[t, 1] == pytest.approx(0.3 * s - 1.2 * c, abs=1e-15)


def test_rope_frequencies_and_pairing():
    """hd = 4, base b: dims (0, 2) turn at angle t, dims (1, 3) at t b^(-1/2)."""
    b = 10000.0
    cos, sin = MM.rope_tables(7, 4, b)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 4))
    out = MM.rope_fwd(x, cos, sin)
    for t in range(7):
        for (i, j, w) in ((0, 2, 1.0), (1, 3, b ** -0.5)):
            c, s = math.cos(t * w), math.sin(t * w)
            assert out[t, i] == pytest.approx(x[t, i] * c - x[t, j] * s, abs=1e-14)
            assert out[t, j] == pytest.approx(x[t, j] * c + x[t, i] * s, abs=1e-14)


def test_rope_relative_position_and_norm():
    """The score of a rotated query and key depends on positions only through
    their difference, and the rotation keeps norms."""
    hd, T = 64, 40
    cos, sin = MM.rope_tables(T, hd)
    rng = np.random.default_rng(2)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    Q = MM.rope_fwd(np.tile(q, (T, 1)), cos, sin)
    K = MM.rope_fwd(np.tile(k, (T, 1)), cos, sin)
    for (t, s, d) in ((5, 2, 7), (30, 30, 9), (3, 17, 20)):
        assert Q[t] @ K[s] == pytest.approx(Q[t + d] @ K[s + d], rel=1e-10, abs=1e-10)
    np.testing.assert_allclose(np.linalg.norm(Q, axis=1), np.linalg.norm(q), rtol=1e-12)
    np.testing.assert_allclose(Q[0], q, rtol=0, atol=0)


def test_rope_backward_is_the_transpose():
    cos, sin = MM.rope_tables(9, 8)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 8))
    y = rng.standard_normal((9, 8))
    assert float((MM.rope_fwd(x, cos, sin) * y).sum()) == pytest.approx(float((x * MM.rope_bwd(y, cos, sin)).sum()),
                                                                        rel=1e-12)


# ----------------------------------------------------------------------------
# RMSNorm and SwiGLU
# ----------------------------------------------------------------------------

def test_rmsnorm_invariants():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 32)) * 3 + 0.5
    w = 1 + 0.1 * rng.standard_normal(32)
    y, (xhat, rstd) = MM.rmsnorm_fwd(x, np.ones(32))
    ms = (x * x).mean(axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), ms / (ms + MM.RMS_EPS), rtol=1e-12)
    y2, _ = MM.rmsnorm_fwd(4.0 * x, np.ones(32), eps=0.0)
    y1, _ = MM.rmsnorm_fwd(x, np.ones(32), eps=0.0)
    np.testing.assert_allclose(y2, y1, rtol=1e-13)
    # sum_i dx_i x_i = eps / (ms + eps) * sum_i g_i xhat_i  (the chain rule through rstd)
    eps = 0.3
    _, cache = MM.rmsnorm_fwd(x, w, eps=eps)
    dy = rng.standard_normal(x.shape)
    dx, _ = MM.rmsnorm_bwd(dy, cache, w)
    g = dy * w
    np.testing.assert_allclose((dx * x).sum(axis=1), eps / (ms + eps) * (g * cache[0]).sum(axis=1), rtol=1e-10)


def test_rmsnorm_and_silu_against_torch():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 24))
    w = 1 + 0.1 * rng.standard_normal(24)
    y, _ = MM.rmsnorm_fwd(x, w)
    ref = F.rms_norm(torch.tensor(x), (24,), torch.tensor(w), eps=MM.RMS_EPS).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12)
    g = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(MM.silu(g), F.silu(torch.tensor(g)).numpy(), rtol=1e-12)
    gt = torch.tensor(g, requires_grad=True)
    F.silu(gt).sum().backward()
    np.testing.assert_allclose(MM.silu_grad(g), gt.grad.numpy(), rtol=1e-12)
    assert MM.silu(np.array(0.0)) == 0.0
    assert MM.silu_grad(np.array(0.0)) == 0.5


def test_against_torch_cpu_autograd():
    """The whole variant written with PyTorch CPU routines (rms_norm, SDPA,
    silu, cross_entropy) and differentiated by autograd, in float64."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    cfg = MM.ModernConfig(vocab_size=40, block_size=16, n_layer=2, n_head=4, n_embd=32, mlp_hidden=48)
    params = {k: v.astype(np.float64)
              for k, v in synthetic.random_params(MM.param_specs(cfg), seed=12, matrix_std=0.1).items()}
    rng = np.random.default_rng(13)
    x = rng.integers(0, cfg.vocab_size, size=(3, 16))
    y = rng.integers(0, cfg.vocab_size, size=(3, 16))
    y[0, :2] = -1
    scale = 0.25
    loss, _, g = MM.fwd_bwd(cfg, params, x, y, scale=scale)

    tp = {k: torch.tensor(v, requires_grad=True) for k, v in params.items()}
    X = torch.tensor(x, dtype=torch.long)
    Y = torch.tensor(y, dtype=torch.long)
    B, T = x.shape
    C, H, Fh = cfg.n_embd, cfg.n_head, cfg.mlp_hidden
    hd = C // H
    inv = 1.0 / (cfg.rope_base ** (torch.arange(0, hd, 2, dtype=torch.float64) / hd))
    ang = torch.outer(torch.arange(T, dtype=torch.float64), inv)
    cos = torch.cat([ang, ang], dim=-1).cos()
    sin = torch.cat([ang, ang], dim=-1).sin()

    def rot(t):
        t1, t2 = t[..., :hd // 2], t[..., hd // 2:]
        return t * cos + torch.cat([-t2, t1], dim=-1) * sin

    h = tp["transformer.wte.weight"][X]
    eps = MM.RMS_EPS
    for layer in range(cfg.n_layer):
        p = f"transformer.h.{layer}."
        a = F.rms_norm(h, (C,), tp[p + "ln_1.weight"], eps=eps)
        q, k, v = F.linear(a, tp[p + "attn.c_attn.weight"]).split(C, dim=2)
        q, k, v = (t.view(B, T, H, hd).transpose(1, 2) for t in (q, k, v))
        o = F.scaled_dot_product_attention(rot(q), rot(k), v, is_causal=True)
        h = h + F.linear(o.transpose(1, 2).reshape(B, T, C), tp[p + "attn.c_proj.weight"])
        a = F.rms_norm(h, (C,), tp[p + "ln_2.weight"], eps=eps)
        gate, up = F.linear(a, tp[p + "mlp.c_fc.weight"]).split(Fh, dim=2)
        h = h + F.linear(F.silu(gate) * up, tp[p + "mlp.c_proj.weight"])
    z = F.rms_norm(h, (C,), tp["transformer.ln_f.weight"], eps=eps)
    logits = z @ tp["transformer.wte.weight"].T
    tl = F.cross_entropy(logits.view(-1, cfg.vocab_size), Y.view(-1), ignore_index=-1)
    (tl * scale).backward()
    assert float(tl) == pytest.approx(loss, rel=1e-12)
    for name in params:
        np.testing.assert_allclose(g[name], tp[name].grad.numpy(), rtol=1e-8, atol=1e-13, err_msg=name)


def test_shares_attention_and_loss_with_the_gpt2_oracle():
    """The variant reuses the oracle's attention and cross-entropy; a model
    whose RoPE angles are all zero (T = 1) reduces attention to o = v."""
    cos, sin = MM.rope_tables(1, 8)
    assert np.array_equal(cos, np.ones((1, 8))) and np.array_equal(sin, np.zeros((1, 8)))
    v = np.arange(8.0)[None, :]
    o, p = M.attention_fwd(np.ones((1, 8)), np.ones((1, 8)), v)
    np.testing.assert_array_equal(o, v)
