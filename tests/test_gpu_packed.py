"""Packed windows under a document mask on the GPU ("GPT" chapter of Zero to
Frontier, "Document boundaries, packing and masking"), through the C-ABI,
against the oracle's packed path (oracle.model.packed_mask / forward(eot=)).

* gpt2_op_segment_starts: bit-exact against the oracle's positions;
* gpt2_op_attention_fwd / _bwd with document starts: against the oracle's
  masked attention on the same inputs, rows with documents at tile edges,
  consecutive separators, a separator as the last token and a row made only
  of separators;
* the whole micro-step with gpt2_set_doc_mask: float32 mode to the float32
  bars, bf16 mode (GPT-2 and the rotary variant, and GPT-2 124M at its real
  width) to the bf16 bars; a captured graph keeps the mask; switching the
  mask off gives back the plain model.

Inputs: the synthetic token stream (a separator before every document) with
short documents, so that every window holds several of them.
"""

import numpy as np
import pytest

from gpu_util import announce, bf16_round, cosine, dev, host, load_params, read_named, rel_l2
from oracle import model as OM
from oracle import modern as OMM
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    import gpt_pretraining_step_amd as g
    assert torch.cuda.is_available()
    g.lib()
    return g


def packed_tokens(B, T, eot, mean_doc, seed, force=()):
    """[B, T] int32 windows cut from a stream with a separator before each
    document (ids below ``eot``, separator ``eot``); ``force`` lists
    (row, position) pairs that are set to the separator."""
    s = synthetic.token_stream(B * T, seed=seed, vocab=eot, eot=eot, mean_doc=mean_doc)
    x = s.reshape(B, T).copy()
    for b, t in force:
        if t < T:
            x[b, t] = eot
    return x.astype(np.int32)


EDGES = [(0, 0), (0, 63), (0, 64), (0, 127), (0, 128), (0, 129), (0, 300), (0, 301), (0, 1023)]


# ---------------------------------------------------------------- segments

@pytest.mark.parametrize("B,T", [(1, 1), (3, 100), (2, 256), (2, 1000), (4, 1024)])
def test_segment_starts_exact(g, B, T):
    announce(f"segment starts B={B} T={T}")
    E = 777
    x = packed_tokens(B, T, E, 60, seed=T + B, force=[(0, t) for _, t in EDGES] + [(B - 1, T - 1)])
    if B > 2:
        x[1] = 5          # a row without separator
        x[2] = E          # a row of separators only
    got = host(g.op_segment_starts(dev(x), E))
    _, pos = OM.packed_rows(x, E)
    assert np.array_equal(got, np.arange(T)[None, :] - pos)


# ---------------------------------------------------------------- attention

def _attn_oracle_masked(qkv, B, T, H, hd, dy, masks):
    C = H * hd
    y = np.zeros((B, T, C))
    lse = np.zeros((B, H, T))
    dqkv = np.zeros((B, T, 3 * C))
    q3 = qkv.reshape(B, T, 3, H, hd).astype(np.float64)
    for b in range(B):
        for h in range(H):
            q, k, v = q3[b, :, 0, h], q3[b, :, 1, h], q3[b, :, 2, h]
            o, p = OM.attention_fwd(q, k, v, masks[b])
            y[b, :, h * hd:(h + 1) * hd] = o
            s = (q @ k.T) / np.sqrt(hd)
            s[~masks[b]] = -np.inf
            mx = s.max(-1)
            lse[b, h] = mx + np.log(np.exp(s - mx[:, None]).sum(-1))
            do = dy[b, :, h * hd:(h + 1) * hd].astype(np.float64)
            dq, dk, dv = OM.attention_bwd(do, q, k, v, p)
            dqkv[b, :, h * hd:(h + 1) * hd] = dq
            dqkv[b, :, C + h * hd:C + (h + 1) * hd] = dk
            dqkv[b, :, 2 * C + h * hd:2 * C + (h + 1) * hd] = dv
    return y, lse, dqkv


@pytest.mark.parametrize("B,T,H,mean_doc", [(2, 1024, 2, 150), (1, 300, 3, 40), (2, 129, 1, 10), (1, 64, 2, 1000)])
def test_attention_bf16_doc_mask_vs_oracle(g, B, T, H, mean_doc):
    import torch
    hd, E = 64, 500
    announce(f"attention bf16 doc mask B={B} T={T} H={H} mean_doc={mean_doc}")
    x = packed_tokens(B, T, E, mean_doc, seed=T + H, force=EDGES)
    masks, _ = OM.packed_rows(x, E)
    rng = np.random.default_rng(T + 7 * H)
    qkv = bf16_round(rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32))
    dy = bf16_round(rng.standard_normal((B * T, H * hd)).astype(np.float32))
    y_ref, lse_ref, dqkv_ref = _attn_oracle_masked(qkv, B, T, H, hd, dy.reshape(B, T, -1), masks)
    seg = g.op_segment_starts(dev(x), E)
    dq = dev(qkv, torch.bfloat16)
    y = torch.zeros((B * T, H * hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dq, y, lse, B, T, H, hd, seg=seg)
    yh = host(y).reshape(B, T, -1)
    assert cosine(yh, y_ref) > 0.9999
    assert np.abs(yh - y_ref).max() <= 2e-2 * max(1.0, np.abs(y_ref).max())
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-4, atol=1e-3)
    dqkv = torch.zeros((B * T, 3 * H * hd), dtype=torch.bfloat16, device="cuda")
    g.op_attention_bwd(dq, y, dev(dy, torch.bfloat16), lse, dqkv, B, T, H, hd, seg=seg)
    got = host(dqkv).reshape(B, T, 3, H, hd)
    ref = dqkv_ref.reshape(B, T, 3, H, hd)
    for part, name in ((0, "dq"), (1, "dk"), (2, "dv")):
        assert cosine(got[:, :, part], ref[:, :, part]) > 0.999, name
        assert np.abs(got[:, :, part] - ref[:, :, part]).max() <= 3e-2 * max(1.0, np.abs(ref[:, :, part]).max()), name


def test_attention_bf16_every_token_a_document(g):
    """A row of separators only: each query sees only itself, so y = v and
    dv = dy exactly (the one probability rounds to 1 in bf16), and dq = dk = 0
    up to the rounding of dO.v - rowsum(dO o O)."""
    import torch
    B, T, H, hd, E = 1, 200, 2, 64, 3
    announce("attention bf16 doc mask, one-token documents")
    x = np.full((B, T), E, dtype=np.int32)
    rng = np.random.default_rng(2)
    qkv = bf16_round(rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32))
    dy = bf16_round(rng.standard_normal((B * T, H * hd)).astype(np.float32))
    seg = g.op_segment_starts(dev(x), E)
    dq = dev(qkv, torch.bfloat16)
    y = torch.zeros((B * T, H * hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dq, y, lse, B, T, H, hd, seg=seg)
    C = H * hd
    assert np.array_equal(host(y), qkv[:, 2 * C:])
    dqkv = torch.full((B * T, 3 * C), 7.0, dtype=torch.bfloat16, device="cuda")
    g.op_attention_bwd(dq, y, dev(dy, torch.bfloat16), lse, dqkv, B, T, H, hd, seg=seg)
    got = host(dqkv)
    assert np.abs(got[:, :2 * C]).max() <= 1e-3
    assert np.array_equal(got[:, 2 * C:], dy)


@pytest.mark.parametrize("B,T,H,hd", [(2, 100, 2, 16), (1, 70, 3, 64)])
def test_attention_fp32_doc_mask_vs_oracle(g, B, T, H, hd):
    announce(f"attention fp32 doc mask B={B} T={T} H={H} hd={hd}")
    E = 30
    x = packed_tokens(B, T, E, 12, seed=T, force=[(0, 0), (0, 1), (0, T - 1)])
    masks, _ = OM.packed_rows(x, E)
    rng = np.random.default_rng(9)
    qkv = rng.standard_normal((B * T, 3 * H * hd)).astype(np.float32)
    dy = rng.standard_normal((B * T, H * hd)).astype(np.float32)
    y_ref, lse_ref, dqkv_ref = _attn_oracle_masked(qkv, B, T, H, hd, dy.reshape(B, T, -1), masks)
    import torch
    seg = g.op_segment_starts(dev(x), E)
    y = torch.zeros((B * T, H * hd), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dev(qkv), y, lse, B, T, H, hd, seg=seg)
    np.testing.assert_allclose(host(y).reshape(B, T, -1), y_ref, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-5, atol=1e-5)
    dqkv = torch.zeros((B * T, 3 * H * hd), dtype=torch.float32, device="cuda")
    g.op_attention_bwd(dev(qkv), y, dev(dy), lse, dqkv, B, T, H, hd, seg=seg)
    np.testing.assert_allclose(host(dqkv).reshape(B, T, -1), dqkv_ref.reshape(B, T, -1), rtol=1e-4, atol=1e-4)


# ---------------------------------------------------------------- whole step

def ocfg(c):
    return OM.Config(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


def ocfg_rot(c):
    return OMM.ModernConfig(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


def _step(g, m, x, y, scale):
    import torch
    tl = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    loss = m.fwd_bwd(dev(x), dev(y), loss_scale=scale, token_loss=tl)
    assert m.status() == 0
    return float(host(loss)[0]), host(tl), read_named(m, m.grads)


def _windows(B, T, vocab, eot, mean_doc, seed):
    s = synthetic.token_stream(B * T + 1, seed=seed, vocab=vocab, eot=eot, mean_doc=mean_doc)
    return synthetic.micro_batch(s, 0, B, T)


def test_tiny_fp32_doc_mask_step_parity(g):
    cfg = g.TINY_CHAR_FP32
    oc = ocfg(cfg)
    E = cfg.vocab_size - 1
    announce("tiny fp32 fwd_bwd with the document mask")
    m = g.GPT2(cfg)
    params = synthetic.random_params(OM.param_specs(oc), seed=5)
    load_params(m, params)
    m.zero_grad()
    m.set_doc_mask(E)
    x, y = _windows(4, 64, E, E, 12, seed=3)
    assert (x == E).sum() >= 8
    loss, tl, grads = _step(g, m, x, y, 1.0)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    lref, rl, gref = OM.fwd_bwd(oc, p64, x, y, eot=E)
    assert abs(loss - lref) / abs(lref) <= 1e-4
    np.testing.assert_allclose(tl.reshape(-1), rl, rtol=1e-4, atol=1e-5)
    worst = max((rel_l2(grads[n], gref[n]), n) for n in gref if np.linalg.norm(gref[n]) > 0)
    assert worst[0] <= 1e-3, worst
    # positions no window reaches get no gradient
    _, pos = OM.packed_rows(x, E)
    unreached = sorted(set(range(cfg.block_size)) - set(pos.reshape(-1).tolist()))
    assert unreached and np.abs(grads["transformer.wpe.weight"][unreached]).max() == 0.0
    m.close()


SMALL_BF16 = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=2, n_embd=128, mlp_hidden=512)
SMALL_ROT = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=4, n_embd=256, mlp_hidden=160)


@pytest.mark.parametrize("arch", ["gpt2", "rotary"])
def test_small_bf16_doc_mask_step_parity(g, arch):
    rot = arch == "rotary"
    cfg = g.ModelConfig(**(SMALL_ROT if rot else SMALL_BF16), max_batch=3, precision=g.PRECISION_BF16,
                        arch=g.ARCH_ROTARY if rot else g.ARCH_GPT2)
    E = cfg.vocab_size - 1
    announce(f"small bf16 {arch} fwd_bwd with the document mask B=3 T=200")
    oc, mod = (ocfg_rot(cfg), OMM) if rot else (ocfg(cfg), OM)
    m = g.GPT2(cfg)
    params = synthetic.random_params(mod.param_specs(oc), seed=21)
    load_params(m, params)
    m.zero_grad()
    m.set_doc_mask(E)
    x, y = _windows(3, 200, E, E, 40, seed=4)
    x[0, [0, 63, 64, 127, 128]] = E
    loss, tl, grads = _step(g, m, x, y, 0.5)
    lref, rl, gref = mod.fwd_bwd(oc, params, x, y, scale=0.5, eot=E)
    assert abs(loss - lref) / abs(lref) <= 1e-2
    assert np.abs(tl.reshape(-1) - rl).max() <= 0.05
    for k in gref:
        if np.linalg.norm(gref[k]) > 0:
            c = cosine(grads[k], gref[k])
            assert c >= 0.999, (k, c)
    # the mask matters at these sizes: the plain causal gradients are further off
    gplain = mod.fwd_bwd(oc, params, x, y, scale=0.5)[2]
    k = "transformer.h.0.attn.c_attn.weight"
    assert rel_l2(grads[k], gref[k]) < 0.5 * rel_l2(grads[k], gplain[k])
    m.close()


@pytest.mark.timeout(600)
def test_gpt2_124m_bf16_doc_mask_step_parity_b1(g):
    """GPT-2 124M at its real width, one packed window of 1024 tokens with
    documents of mean length 150: loss and every gradient tensor against the
    float32 oracle."""
    cfg = g.ModelConfig(50304, 1024, 12, 12, 768, 3072, 1, g.PRECISION_BF16)
    oc = ocfg(cfg)
    E = synthetic.EOT_ID
    announce("gpt2-124m bf16 fwd_bwd with the document mask B=1 T=1024")
    m = g.GPT2(cfg)
    params = synthetic.random_params(OM.param_specs(oc), seed=42)
    load_params(m, params)
    m.zero_grad()
    m.set_doc_mask(E)
    x, y = _windows(1, 1024, synthetic.GPT2_VOCAB, E, 150, seed=6)
    assert (x == E).sum() >= 3
    loss, tl, grads = _step(g, m, x, y, 0.5)
    m.close()
    lref, rl, gref = OM.fwd_bwd(oc, params, x, y, scale=0.5, eot=E)
    assert abs(loss - lref) / abs(lref) <= 1e-2
    worst = min((cosine(grads[k], gref[k]), k) for k in gref if np.linalg.norm(gref[k]) > 0)
    assert worst[0] >= 0.999, worst


def test_doc_mask_setting_graph_and_switch_off(g):
    import torch
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=2, precision=g.PRECISION_BF16)
    E = cfg.vocab_size - 1
    announce("doc mask: argument checks, graph capture, switching off")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(OM.param_specs(ocfg(cfg)), seed=8))
    for bad in (-2, cfg.vocab_size):
        with pytest.raises(g.GPT2Error) as e:
            m.set_doc_mask(bad)
        assert e.value.status == g._ffi.GPT2_ERR_ARG
    x, y = _windows(2, 128, E, E, 30, seed=5)
    # the plain model first, then the masked one (they differ)
    m.zero_grad()
    l_plain, _, g_plain = _step(g, m, x, y, 1.0)
    m.set_doc_mask(E)
    m.zero_grad()
    l_doc, _, g_doc = _step(g, m, x, y, 1.0)
    assert rel_l2(g_doc["transformer.wpe.weight"], g_plain["transformer.wpe.weight"]) > 0.1
    assert rel_l2(g_doc["transformer.h.0.attn.c_attn.weight"], g_plain["transformer.h.0.attn.c_attn.weight"]) > 0.05
    # a graph captured with the mask replays it
    tok, tgt = dev(x), dev(y)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    m.graph_capture(tok, tgt, loss_scale=1.0, loss_out=loss)
    for _ in range(2):
        m.zero_grad()
        m.graph_launch()
        torch.cuda.synchronize()
        assert m.status() == 0
        assert float(host(loss)[0]) == pytest.approx(l_doc, rel=1e-6)
        got = read_named(m, m.grads)
        for k in got:
            np.testing.assert_allclose(got[k], g_doc[k], rtol=1e-4, atol=1e-6, err_msg=k)
    # changing the setting discards the graph; off gives the plain model back
    m.set_doc_mask(None)
    with pytest.raises(g.GPT2Error) as e:
        m.graph_launch()
    assert e.value.status == g._ffi.GPT2_ERR_UNBOUND
    m.zero_grad()
    l_again, _, g_again = _step(g, m, x, y, 1.0)
    assert l_again == pytest.approx(l_plain, rel=1e-6)
    for k in g_again:
        np.testing.assert_allclose(g_again[k], g_plain[k], rtol=1e-5, atol=1e-7, err_msg=k)
    m.close()
