"""Kernel-level parity on the GPU, through the C-ABI single-op entry points.

GEMM: bit-exact on small-integer operands (every product and partial sum is an
integer below 2^24, so float32 accumulation is exact in any order), in every
operand layout and on shapes that span several tiles with ragged tails; the
fused epilogues against NumPy.  Attention, LayerNorm and the lm_head loss
against the oracle on the same bf16-rounded inputs.
"""

import math

import numpy as np
import pytest

from gpu_util import announce, bf16_round, cosine, dev, host, rel_l2
import oracle
from oracle import model as OM
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    import gpt_pretraining_step_amd as g
    assert torch.cuda.is_available()
    g.lib()
    return g


def _stored(mat_mk, kmajor):
    """A logical [rows, K] operand stored K-major ([rows][K]) or not ([K][rows])."""
    return np.ascontiguousarray(mat_mk if kmajor else mat_mk.T)


LAYOUTS = [(True, True), (True, False), (False, True), (False, False)]
SHAPES = [(8, 8, 16), (200, 136, 72), (520, 392, 200), (136, 264, 1000)]


@pytest.mark.parametrize("ak,bk", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_bf16_integer_exact(g, ak, bk, M, N, K):
    import torch
    announce(f"gemm bf16 int M={M} N={N} K={K} ak={ak} bk={bk}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    ref = (A.astype(np.int64) @ B.astype(np.int64).T).astype(np.float32)
    dA = dev(_stored(A, ak), torch.bfloat16)
    dB = dev(_stored(B, bk), torch.bfloat16)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    g.op_gemm(dA, dB, C, M, N, K, a_kmajor=ak, b_kmajor=bk)
    assert np.array_equal(host(C), ref)


@pytest.mark.parametrize("ak,bk", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_fp32_mfma_integer_exact(g, ak, bk, M, N, K):
    """The float32 mode's product (float32 MFMA on 64x64 tiles): exact on
    small integers in every layout, over ragged tiles and K steps, with the
    residual epilogue on top."""
    import torch
    announce(f"gemm fp32 int M={M} N={N} K={K} ak={ak} bk={bk}")
    rng = np.random.default_rng(M * 5 + N * 11 + K)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    R = rng.integers(-50, 51, size=(M, N)).astype(np.float32)
    ref = (A.astype(np.int64) @ B.astype(np.int64).T).astype(np.float32)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    g.op_gemm(dev(_stored(A, ak)), dev(_stored(B, bk)), C, M, N, K, a_kmajor=ak, b_kmajor=bk)
    assert np.array_equal(host(C), ref)
    g.op_gemm(dev(_stored(A, ak)), dev(_stored(B, bk)), C, M, N, K, a_kmajor=ak, b_kmajor=bk,
              epilogue=g.EPI_RESIDUAL, R=dev(R))
    assert np.array_equal(host(C), ref + R)


def test_gemm_bf16_integer_exact_large_tiles(g):
    import torch
    M, N, K = 4096, 8192, 64  # >= 1024 tiles of 256x128: the large-tile kernel
    announce(f"gemm bf16 int large M={M} N={N} K={K}")
    rng = np.random.default_rng(1)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    ref = (A.astype(np.int64) @ B.astype(np.int64).T).astype(np.float32)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    g.op_gemm(dev(A, torch.bfloat16), dev(B, torch.bfloat16), C, M, N, K)
    assert np.array_equal(host(C), ref)
    for ak, bk in LAYOUTS[1:]:
        C.zero_()
        g.op_gemm(dev(_stored(A, ak), torch.bfloat16), dev(_stored(B, bk), torch.bfloat16), C, M, N, K,
                  a_kmajor=ak, b_kmajor=bk)
        assert np.array_equal(host(C), ref), (ak, bk)


@pytest.mark.parametrize("K", [128, 384, 200])
def test_gemm_bf16_many_tiles_exact(g, K):
    """More output tiles than compute units (several rounds of blocks), ragged
    M and N so that edge tiles sit between interior ones, even and odd K step
    counts: the float32 store and the residual epilogue stay exact on integer
    operands, in all four operand layouts."""
    import torch
    M, N = 4104, 4136
    announce(f"gemm bf16 many tiles M={M} N={N} K={K}")
    rng = np.random.default_rng(K)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    R = rng.integers(-50, 51, size=(M, N)).astype(np.float32)
    ref = (A.astype(np.int64) @ B.astype(np.int64).T).astype(np.float32)
    dR = dev(R)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    for ak, bk in LAYOUTS:
        dA, dB = dev(_stored(A, ak), torch.bfloat16), dev(_stored(B, bk), torch.bfloat16)
        C.fill_(7.0)
        g.op_gemm(dA, dB, C, M, N, K, a_kmajor=ak, b_kmajor=bk)
        assert np.array_equal(host(C), ref), ("store", ak, bk)
        C.fill_(7.0)
        g.op_gemm(dA, dB, C, M, N, K, a_kmajor=ak, b_kmajor=bk, epilogue=g.EPI_RESIDUAL, R=dR)
        assert np.array_equal(host(C), ref + R), ("residual", ak, bk)


def test_gemm_grouped_exact(g):
    """Weight-gradient products of different shapes in one launch (K-slow
    operands, ragged edge tiles, one tiny product): on integer operands
    C += alpha A^T B and the bias row sums stay exact, and every product
    lands in its own output."""
    import torch
    shapes = [(768, 3072, 1024, True, 1.0), (3072, 768, 1024, True, 0.5), (264, 136, 520, False, 1.0),
              (8, 16, 64, True, 2.0), (2304, 776, 1032, True, 1.0)]
    announce(f"gemm grouped {len(shapes)} products")
    rng = np.random.default_rng(5)
    items, refs = [], []
    for M, N, K, with_rs, alpha in shapes:
        A = rng.integers(-4, 5, size=(K, M)).astype(np.float32)  # stored [K][M]
        B = rng.integers(-4, 5, size=(K, N)).astype(np.float32)
        C0 = rng.integers(-100, 101, size=(M, N)).astype(np.float32)
        r0 = rng.integers(-100, 101, size=M).astype(np.float32)
        refC = C0 + alpha * (A.astype(np.int64).T @ B.astype(np.int64)).astype(np.float64)
        refR = r0 + alpha * A.astype(np.int64).sum(axis=0) if with_rs else None
        C, R = dev(C0), (dev(r0) if with_rs else None)
        items.append((dev(A, torch.bfloat16), dev(B, torch.bfloat16), C, M, N, K, R, alpha))
        refs.append((C, refC, R, refR))
    g.op_gemm_grouped(items)
    for i, (C, refC, R, refR) in enumerate(refs):
        assert np.array_equal(host(C), refC.astype(np.float32)), i
        if R is not None:
            assert np.array_equal(host(R), refR.astype(np.float32)), i


@pytest.mark.parametrize("K", [2048, 4096])
def test_gemm_grouped_split_tail_exact(g, K):
    """276 output tiles: one full round of 256 blocks and a 20-tile tail.  At
    K = 4096 the last product runs split in K (four quarters adding
    atomically); at K = 2048 its pieces would be too short and it runs
    whole.  Every output and row sum stays exact on integer operands."""
    import torch
    shapes = [(2048, 2048)] * 4 + [(1024, 1280)]
    announce(f"gemm grouped split tail {len(shapes)} products K={K}")
    rng = np.random.default_rng(6)
    items, refs = [], []
    for idx, (M, N) in enumerate(shapes):
        A = rng.integers(-3, 4, size=(K, M)).astype(np.float32)
        B = rng.integers(-3, 4, size=(K, N)).astype(np.float32)
        C0 = rng.integers(-100, 101, size=(M, N)).astype(np.float32)
        r0 = rng.integers(-100, 101, size=M).astype(np.float32)
        # float64 products of integers below 2^53: exact (and BLAS-fast)
        refC = C0 + A.astype(np.float64).T @ B.astype(np.float64)
        refR = r0 + A.astype(np.float64).sum(axis=0)
        C, R = dev(C0), dev(r0)
        items.append((dev(A, torch.bfloat16), dev(B, torch.bfloat16), C, M, N, K, R, 1.0))
        refs.append((C, refC, R, refR))
    g.op_gemm_grouped(items)
    for i, (C, refC, R, refR) in enumerate(refs):
        assert np.array_equal(host(C), refC.astype(np.float32)), i
        assert np.array_equal(host(R), refR.astype(np.float32)), i


@pytest.mark.parametrize("ak,bk", LAYOUTS)
def test_gemm_bf16_accumulate_split_k_exact(g, ak, bk):
    """Few output tiles and a long K take the split-K path (atomic adds of
    integer partial sums: still exact)."""
    import torch
    M, N, K = 256, 264, 16384
    announce(f"gemm bf16 accumulate split-K M={M} N={N} K={K} ak={ak} bk={bk}")
    rng = np.random.default_rng(2)
    A = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    B = rng.integers(-2, 3, size=(N, K)).astype(np.float32)
    C0 = rng.integers(-100, 100, size=(M, N)).astype(np.float32)
    ref = C0 + (A.astype(np.int64) @ B.astype(np.int64).T).astype(np.float32)
    C = dev(C0)
    g.op_gemm(dev(_stored(A, ak), torch.bfloat16), dev(_stored(B, bk), torch.bfloat16), C, M, N, K,
              a_kmajor=ak, b_kmajor=bk, epilogue=g.EPI_ACCUMULATE)
    assert np.array_equal(host(C), ref)


@pytest.mark.parametrize("M,N,K", [(264, 392, 328), (776, 520, 200), (4096, 4096, 72)])
def test_gemm_bf16_epilogues(g, M, N, K):
    """Every fused epilogue, on tiles wholly inside C (the unchecked store
    path) and on ragged edge tiles; the small shapes take 256x192 block
    tiles, 4096 x 4096 the 256x256 ones."""
    import torch
    announce(f"gemm bf16 epilogues M={M} N={N} K={K}")
    rng = np.random.default_rng(3)
    A = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    B = bf16_round((rng.standard_normal((N, K)) * 0.1).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32)
    R = rng.standard_normal((M, N)).astype(np.float32)
    acc = A.astype(np.float64) @ B.astype(np.float64).T
    v = 0.75 * acc + bias
    dA, dB = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    # STORE bf16 with alpha and bias
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dA, dB, C, M, N, K, bias=dev(bias), alpha=0.75)
    np.testing.assert_allclose(host(C), v, rtol=1e-2, atol=1e-2)
    # RESIDUAL (float32)
    C32 = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    g.op_gemm(dA, dB, C32, M, N, K, bias=dev(bias), alpha=0.75, epilogue=g.EPI_RESIDUAL, R=dev(R))
    np.testing.assert_allclose(host(C32), R + v, rtol=1e-5, atol=1e-4)
    # GELU: U = bf16(v), G = bf16(gelu(U))
    U = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    G = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dA, dB, U, M, N, K, bias=dev(bias), alpha=0.75, epilogue=g.EPI_GELU, C2=G)
    u = host(U)
    np.testing.assert_allclose(u, v, rtol=1e-2, atol=1e-2)
    np.testing.assert_allclose(host(G), OM.gelu_tanh(u.astype(np.float64)), rtol=1e-2, atol=1e-2)
    # DGELU: out = bf16(v * gelu'(U))
    D = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dA, dB, D, M, N, K, alpha=0.75, epilogue=g.EPI_DGELU, U=U)
    ref = 0.75 * acc * OM.gelu_tanh_grad(u.astype(np.float64))
    np.testing.assert_allclose(host(D), ref, rtol=2e-2, atol=2e-2)
    # GELU_GRAD: u = bf16(v); C = bf16(gelu(u)), C2 = bf16(gelu'(u))
    Gg = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    Gd = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dA, dB, Gg, M, N, K, bias=dev(bias), alpha=0.75, epilogue=g.EPI_GELU_GRAD, C2=Gd)
    np.testing.assert_allclose(host(Gg), OM.gelu_tanh(u.astype(np.float64)), rtol=1e-2, atol=1e-2)
    gd = host(Gd)
    np.testing.assert_allclose(gd, OM.gelu_tanh_grad(u.astype(np.float64)), rtol=1e-2, atol=1e-2)
    # MUL: out = bf16(v * U), here with U = gelu'(u): the backward's dGELU
    P = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g.op_gemm(dA, dB, P, M, N, K, alpha=0.75, epilogue=g.EPI_MUL, U=Gd)
    np.testing.assert_allclose(host(P), 0.75 * acc * gd.astype(np.float64), rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("ak,bk", LAYOUTS)
def test_gemm_fp32_all_layouts(g, ak, bk):
    import torch
    M, N, K = 70, 66, 130
    announce(f"gemm fp32 M={M} N={N} K={K} ak={ak} bk={bk}")
    rng = np.random.default_rng(4)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    g.op_gemm(dev(_stored(A, ak)), dev(_stored(B, bk)), C, M, N, K, a_kmajor=ak, b_kmajor=bk)
    np.testing.assert_allclose(host(C), ref, rtol=1e-5, atol=1e-4)
    C2 = dev(np.ones((M, N), dtype=np.float32))
    g.op_gemm(dev(_stored(A, ak)), dev(_stored(B, bk)), C2, M, N, K, a_kmajor=ak, b_kmajor=bk,
              epilogue=g.EPI_ACCUMULATE)
    np.testing.assert_allclose(host(C2), 1 + ref, rtol=1e-5, atol=1e-4)


def test_gemm_rejects_bad_arguments(g):
    import torch
    announce("gemm argument checks")
    A = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, A, C, 16, 16, 12)          # K not a multiple of 8 for bf16 K-major operands
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, A, C, 16, 16, 16, lda=8)   # pitch smaller than K
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, A, C, 16, 16, 16, epilogue=g.EPI_RESIDUAL)  # residual without R
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, A, C, 16, 16, 16, epilogue=g.EPI_MUL)  # product without U
    with pytest.raises(g.GPT2Error):
        g.op_gemm(A, A, C, 16, 16, 16, epilogue=g.EPI_MUL, U=A)  # bf16 product into a float32 C


def test_colsum(g):
    import torch
    announce("colsum")
    rng = np.random.default_rng(5)
    Y = bf16_round(rng.standard_normal((1000, 200)).astype(np.float32))
    db = dev(np.ones(200, dtype=np.float32))
    g.op_colsum(dev(Y, torch.bfloat16), db)
    np.testing.assert_allclose(host(db), 1 + Y.astype(np.float64).sum(0), rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------ attention

def _attn_oracle(qkv, B, T, H, hd, dy=None):
    C = H * hd
    y = np.zeros((B, T, C))
    lse = np.zeros((B, H, T))
    dqkv = np.zeros((B, T, 3 * C)) if dy is not None else None
    q3 = qkv.reshape(B, T, 3, H, hd).astype(np.float64)
    for b in range(B):
        for h in range(H):
            q, k, v = q3[b, :, 0, h], q3[b, :, 1, h], q3[b, :, 2, h]
            o, p = OM.attention_fwd(q, k, v)
            y[b, :, h * hd:(h + 1) * hd] = o
            s = (q @ k.T) / math.sqrt(hd)
            s[np.triu(np.ones((T, T), dtype=bool), 1)] = -np.inf
            mx = s.max(-1)
            lse[b, h] = mx + np.log(np.exp(s - mx[:, None]).sum(-1))
            if dy is not None:
                do = dy[b, :, h * hd:(h + 1) * hd].astype(np.float64)
                dq, dk, dv = OM.attention_bwd(do, q, k, v, p)
                dqkv[b, :, h * hd:(h + 1) * hd] = dq
                dqkv[b, :, C + h * hd:C + (h + 1) * hd] = dk
                dqkv[b, :, 2 * C + h * hd:2 * C + (h + 1) * hd] = dv
    return y, lse, dqkv


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 64, 2), (2, 100, 3), (1, 257, 2), (1, 1024, 1)])
def test_attention_bf16_vs_oracle(g, B, T, H):
    import torch
    hd = 64
    announce(f"attention bf16 B={B} T={T} H={H}")
    rng = np.random.default_rng(T + H)
    qkv = bf16_round(rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32))
    dy = bf16_round(rng.standard_normal((B * T, H * hd)).astype(np.float32))
    y_ref, lse_ref, dqkv_ref = _attn_oracle(qkv, B, T, H, hd, dy.reshape(B, T, -1))
    dq = dev(qkv, torch.bfloat16)
    y = torch.zeros((B * T, H * hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dq, y, lse, B, T, H, hd)
    yh = host(y).reshape(B, T, -1)
    assert cosine(yh, y_ref) > 0.9999
    assert np.abs(yh - y_ref).max() <= 2e-2 * max(1.0, np.abs(y_ref).max())
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-4, atol=1e-3)
    if T == 1:
        np.testing.assert_allclose(yh[:, 0], qkv.reshape(B, 3, -1)[:, 2], rtol=1e-2)
    dqkv = torch.zeros((B * T, 3 * H * hd), dtype=torch.bfloat16, device="cuda")
    # the backward consumes the forward's own output and LSE, as in training
    g.op_attention_bwd(dq, y, dev(dy, torch.bfloat16), lse, dqkv, B, T, H, hd)
    got = host(dqkv).reshape(B, T, 3, H, hd)
    ref = dqkv_ref.reshape(B, T, 3, H, hd)
    for part, name in ((0, "dq"), (1, "dk"), (2, "dv")):
        if T == 1 and part < 2:
            assert np.abs(got[:, :, part]).max() <= 5e-2  # one key: no gradient through the softmax (exactly 0 in exact arithmetic)
            continue
        assert cosine(got[:, :, part], ref[:, :, part]) > 0.999, name


@pytest.mark.parametrize("B,T,H,hd", [(2, 64, 4, 16), (1, 37, 2, 64)])
def test_attention_fp32_vs_oracle(g, B, T, H, hd):
    import torch
    announce(f"attention fp32 B={B} T={T} H={H} hd={hd}")
    rng = np.random.default_rng(7)
    qkv = rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32)
    dy = rng.standard_normal((B * T, H * hd)).astype(np.float32)
    y_ref, lse_ref, dqkv_ref = _attn_oracle(qkv, B, T, H, hd, dy.reshape(B, T, -1))
    y = torch.zeros((B * T, H * hd), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dev(qkv), y, lse, B, T, H, hd)
    np.testing.assert_allclose(host(y).reshape(B, T, -1), y_ref, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-5, atol=1e-5)
    dqkv = torch.zeros((B * T, 3 * H * hd), dtype=torch.float32, device="cuda")
    g.op_attention_bwd(dev(qkv), y, dev(dy), lse, dqkv, B, T, H, hd)
    np.testing.assert_allclose(host(dqkv).reshape(B, T, -1), dqkv_ref.reshape(B, T, -1), rtol=1e-4, atol=1e-4)


def test_attention_causality_bitwise(g):
    """Changing keys/values after position t leaves outputs at <= t bitwise
    unchanged (masked products add exact zeros)."""
    import torch
    B, T, H, hd, t = 1, 300, 2, 64, 150
    announce("attention bf16 causality")
    rng = np.random.default_rng(8)
    qkv = bf16_round(rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32))
    qkv2 = qkv.copy()
    qkv2[t + 1:] = bf16_round(rng.standard_normal((T - t - 1, 3 * H * hd)).astype(np.float32))
    outs = []
    for x in (qkv, qkv2):
        y = torch.zeros((B * T, H * hd), dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
        g.op_attention_fwd(dev(x, torch.bfloat16), y, lse, B, T, H, hd)
        outs.append((host(y), host(lse)))
    assert np.array_equal(outs[0][0][:t + 1], outs[1][0][:t + 1])
    assert np.array_equal(outs[0][1][..., :t + 1], outs[1][1][..., :t + 1])
    assert not np.array_equal(outs[0][0][t + 1:], outs[1][0][t + 1:])


# ------------------------------------------------------------------ layernorm

@pytest.mark.parametrize("rows,C,bf,dyb", [(1, 768, True, False), (1000, 768, True, False), (1000, 768, True, True),
                                           (129, 256, True, True), (70, 512, True, False), (65, 1024, True, True),
                                           (77, 64, False, False), (33, 100, False, True)])
def test_layernorm_vs_oracle(g, rows, C, bf, dyb):
    """Forward and backward against the oracle.  C a multiple of 256 takes the
    vector kernels (one float4 group per lane per 256 columns, 16 rows per
    wave in the backward, ragged row counts); other C the generic ones.  dy is
    float32 or bf16 (rounded on the host, so both sides see the same values);
    the bf16 copy of the updated dx must equal bf16 of the float32 dx."""
    import torch
    announce(f"layernorm rows={rows} C={C} bf16={bf} dy_bf16={dyb}")
    rng = np.random.default_rng(rows + C)
    x = (rng.standard_normal((rows, C)) * 2 + 0.5).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    y_ref, cache = OM.layernorm_fwd(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    y = torch.zeros((rows, C), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    mean = torch.zeros(rows, dtype=torch.float32, device="cuda")
    rstd = torch.zeros(rows, dtype=torch.float32, device="cuda")
    dx_ = dev(x)
    g.op_layernorm_fwd(dx_, dev(w), dev(b), y, mean, rstd)
    tol = 1e-2 if bf else 1e-5
    np.testing.assert_allclose(host(y), y_ref, rtol=tol, atol=tol)
    np.testing.assert_allclose(host(rstd), cache[1][:, 0], rtol=1e-5)
    dy = rng.standard_normal((rows, C)).astype(np.float32)
    if dyb:
        dy = synthetic.round_to_bf16(dy)
    dx0 = rng.standard_normal((rows, C)).astype(np.float32)
    dxr, dwr, dbr = OM.layernorm_bwd(dy.astype(np.float64), cache, w.astype(np.float64))
    dx = dev(dx0)
    dxb = torch.zeros((rows, C), dtype=torch.bfloat16, device="cuda")
    dw = dev(np.ones(C, dtype=np.float32))
    db = dev(np.zeros(C, dtype=np.float32))
    g.op_layernorm_bwd(dev(dy, torch.bfloat16) if dyb else dev(dy), dx_, mean, rstd, dev(w), dx, dw, db,
                       dx_bf16=dxb)
    np.testing.assert_allclose(host(dx), dx0 + dxr, rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(host(dw), 1 + dwr, rtol=1e-4, atol=1e-3)
    np.testing.assert_allclose(host(db), dbr, rtol=1e-4, atol=1e-3)
    assert torch.equal(dxb, dx.to(torch.bfloat16))


# ------------------------------------------------------------- lm_head + loss

@pytest.mark.parametrize("M,C,V,wscale", [(300, 64, 1000, 1.0), (5000, 128, 2056, 1.0), (1000, 128, 4096, 16.0),
                                           (20000, 64, 1024, 1.0)])
def test_lmhead_ce_small_vs_oracle(g, M, C, V, wscale):
    """The fused lm_head + loss against the oracle.  wscale = 16 makes logits
    of size ~10 with a peaked softmax: the bf16 logits stored as offsets from
    their tile maximum must still give accurate probabilities.  M = 20000
    runs three row chunks (8192, 8192 and a ragged 3616)."""
    import torch
    announce(f"lmhead_ce M={M} C={C} V={V} wscale={wscale}")
    h, w, t = synthetic.lmhead_inputs(M=M, C=C, V=V, seed=M)
    w = synthetic.round_to_bf16(w * np.float32(wscale))
    t = np.where(t >= 0, t % V, -1).astype(np.int32)
    loss_ref, _, dh_ref, dw_ref = OM.lmhead_ce(h.astype(np.float64), w.astype(np.float64), t)
    dw = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    loss, dh = g.lmhead_ce(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(t), dw)
    assert abs(float(host(loss)[0]) - loss_ref) <= 2e-5 * abs(loss_ref)
    assert cosine(host(dh), dh_ref) > 0.999
    assert cosine(host(dw), dw_ref) > 0.999
    assert np.all(host(dh)[t < 0] == 0)


def test_lmhead_ce_ignore_index(g):
    """ignore_index other than -1: rows whose target equals it are ignored,
    -1 is then an out-of-range target (flagged GPT2_ERR_BAD_ID and ignored
    too), and the result equals the oracle's with that ignore_index."""
    import torch
    announce("lmhead_ce ignore_index 7")
    M, C, V = 3000, 64, 512
    h, w, t = synthetic.lmhead_inputs(M=M, C=C, V=V, seed=9)
    t = np.where(t >= 0, t % V, 7).astype(np.int32)  # the ignored rows now hold 7
    n7 = int((t == 7).sum())
    assert n7 >= 250
    loss_ref, _, dh_ref, dw_ref = OM.lmhead_ce(h.astype(np.float64), w.astype(np.float64), t, ignore_index=7)
    dw = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss, dh = g.lmhead_ce(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(t), dw, flag=flag, ignore_index=7)
    assert abs(float(host(loss)[0]) - loss_ref) <= 2e-5 * abs(loss_ref)
    assert cosine(host(dh), dh_ref) > 0.999 and cosine(host(dw), dw_ref) > 0.999
    assert np.all(host(dh)[t == 7] == 0)
    assert int(host(flag)[0]) == 0
    # the same call with ignore_index 7 and a -1 among the targets: -1 is a
    # bad id now (flagged, its row ignored like the 7s)
    t2 = t.copy()
    t2[5] = -1
    t3 = t.copy()
    t3[5] = 7
    loss_ref3, _, dh_ref3, _ = OM.lmhead_ce(h.astype(np.float64), w.astype(np.float64), t3, ignore_index=7)
    dw.zero_()
    loss2, dh2 = g.lmhead_ce(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(t2), dw, flag=flag, ignore_index=7)
    assert int(host(flag)[0]) == g._ffi.GPT2_ERR_BAD_ID
    assert abs(float(host(loss2)[0]) - loss_ref3) <= 2e-5 * abs(loss_ref3)
    assert np.all(host(dh2)[5] == 0)


def test_lmhead_ce_all_ignored(g):
    import torch
    announce("lmhead_ce all ignored")
    M, C, V = 64, 64, 512
    h, w, _ = synthetic.lmhead_inputs(M=M, C=C, V=V, seed=1)
    t = np.full(M, -1, dtype=np.int32)
    dw = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss, dh = g.lmhead_ce(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(t), dw, flag=flag)
    assert math.isnan(float(host(loss)[0]))
    assert np.all(host(dh) == 0) and np.all(host(dw) == 0)
    assert int(host(flag)[0]) == g._ffi.GPT2_WARN_NO_TARGETS
