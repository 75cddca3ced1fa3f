"""The embedding backward on the GPU (gpt2_op_embedding_bwd, the kernels
gpt2_fwd_bwd runs) against the oracle's scatter-add (oracle.model.embedding_bwd).

The gradient rows and the tables' starting values are integers times 2^-4
small enough that every partial sum is exact in float32, so the GPU result
must equal the oracle's float64 result exactly, whatever the order of the
additions.  With general float values, a second call must give the same
bits (every gradient row sums its rows in a fixed order).

Cases: one row; ragged tiles with C % 4 != 0 (the one-column path); the
benchmarked micro-step (16 x 1024 Zipf tokens, V = 50,304, C = 768), with
and without the document mask; 20 x 1024 rows (more blocks in every radix
pass than the micro-step); a single token id (one run over every tile,
joined from 256 partials); a small vocabulary (one radix digit)."""

import numpy as np
import pytest

from gpu_util import announce
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


def ids_of(kind, B, T, V, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf":
        return synthetic.zipf_ids(rng, B * T, V, perm=rng.permutation(V)).reshape(B, T).astype(np.int32)
    if kind == "stream":  # Zipf documents, each after an EOT id
        return synthetic.token_stream(B * T, seed=seed, vocab=V).reshape(B, T)
    if kind == "one":
        return np.full((B, T), 17 % V, dtype=np.int32)
    return rng.integers(0, V, size=(B, T)).astype(np.int32)


def exact_values(rng, shape):
    return (rng.integers(-8, 9, size=shape) / 16.0).astype(np.float32)


CASES = [  # B, T, C, V, ids, document mask
    (1, 1, 4, 7, "uniform", False),
    (3, 37, 6, 11, "uniform", False),
    (3, 37, 6, 11, "uniform", True),
    (4, 64, 64, 50, "zipf", False),
    (16, 1024, 768, 50304, "zipf", False),
    (16, 1024, 768, 50304, "stream", True),
    (20, 1024, 768, 50304, "zipf", False),
    (20, 1024, 768, 50304, "stream", True),
    (8, 1024, 768, 50304, "one", False),
    (16, 1024, 768, 200, "uniform", False),
]


@pytest.mark.parametrize("B,T,C,V,kind,doc", CASES)
def test_embedding_bwd_exact(g, B, T, C, V, kind, doc):
    import torch
    announce(f"embedding_bwd exact B={B} T={T} C={C} V={V} ids={kind} doc={doc}")
    rng = np.random.default_rng(B * 1000 + T + C + V)
    ids = ids_of(kind, B, T, V, seed=B + T)
    eot = synthetic.EOT_ID if kind == "stream" else int(ids[0, min(T - 1, 3)])
    dh = exact_values(rng, (B, T, C))
    wte0 = exact_values(rng, (V, C))
    wpe0 = exact_values(rng, (T, C))
    tok = torch.from_numpy(ids).cuda()
    seg = g.op_segment_starts(tok, eot) if doc else None
    dwte = torch.from_numpy(wte0).cuda()
    dwpe = torch.from_numpy(wpe0).cuda()
    g.op_embedding_bwd(tok, torch.from_numpy(dh).cuda(), dwte, dwpe, seg=seg)
    torch.cuda.synchronize()
    pos = OM.packed_rows(ids, eot)[1] if doc else None
    ew, ep = OM.embedding_bwd(ids, dh.astype(np.float64), V, T, pos)
    got_w, got_p = dwte.cpu().numpy(), dwpe.cpu().numpy()
    assert np.array_equal(got_w, (wte0 + ew).astype(np.float32)), np.abs(got_w - (wte0 + ew)).max()
    assert np.array_equal(got_p, (wpe0 + ep).astype(np.float32)), np.abs(got_p - (wpe0 + ep)).max()


@pytest.mark.parametrize("B,doc", [(16, False), (16, True), (20, False)])
def test_embedding_bwd_repeatable_bits(g, B, doc):
    import torch
    announce(f"embedding_bwd repeatable B={B} doc={doc}")
    T, C, V = 1024, 768, 50304
    ids = ids_of("stream", B, T, V, seed=5)
    tok = torch.from_numpy(ids).cuda()
    seg = g.op_segment_starts(tok, synthetic.EOT_ID) if doc else None
    gen = torch.Generator().manual_seed(3)
    dres = torch.randn(B * T, C, generator=gen).cuda()
    outs = []
    for _ in range(2):
        dwte = torch.zeros(V, C, device="cuda")
        dwpe = torch.zeros(T, C, device="cuda")
        g.op_embedding_bwd(tok, dres, dwte, dwpe, seg=seg)
        outs.append((dwte.cpu(), dwpe.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # and the values agree with the float64 scatter to float32 rounding
    ew, ep = OM.embedding_bwd(ids, dres.cpu().double().numpy().reshape(B, T, C), V, T,
                              OM.packed_rows(ids, synthetic.EOT_ID)[1] if doc else None)
    scale = np.abs(ew).max()
    assert np.abs(outs[0][0].numpy() - ew).max() <= 1e-5 * scale
    assert np.abs(outs[0][1].numpy() - ep).max() <= 1e-5 * np.abs(ep).max()

