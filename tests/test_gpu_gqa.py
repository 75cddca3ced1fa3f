"""Grouped-query attention on the GPU ("Build an LLM From Scratch: Making
Training Fast on One GPU", step 2: n_head / n_kv_head query heads share each
key/value head), through the C-ABI, against the oracle.

* gpt2_op_attention_fwd / _bwd with Hkv < H, bf16 and float32, with and
  without the document mask: outputs and the gradients of the shared heads
  (summed over their groups) against the oracle's attention run per query
  head on the repeated key/value heads;
* the rotary variant with n_kv_head: a small model and the 124M width (12
  query heads sharing 4 key/value heads, groups of 3 as on that page)
  against oracle.modern to the bf16 bars, and with the document mask.
"""

import numpy as np
import pytest

from gpu_util import announce, bf16_round, cosine, dev, host, load_params, read_named
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


def _oracle(qkv, B, T, H, Hkv, hd, dy, masks):
    C, Ckv, grp = H * hd, Hkv * hd, H // Hkv
    x = qkv.reshape(B, T, -1).astype(np.float64)
    y = np.zeros((B, T, C))
    lse = np.zeros((B, H, T))
    dqkv = np.zeros((B, T, C + 2 * Ckv))
    for b in range(B):
        mask = np.tril(np.ones((T, T), dtype=bool)) if masks is None else masks[b]
        for h in range(H):
            j = h // grp
            q = x[b, :, h * hd:(h + 1) * hd]
            k = x[b, :, C + j * hd:C + (j + 1) * hd]
            v = x[b, :, C + Ckv + j * hd:C + Ckv + (j + 1) * hd]
            o, p = OM.attention_fwd(q, k, v, mask)
            y[b, :, h * hd:(h + 1) * hd] = o
            s = (q @ k.T) / np.sqrt(hd)
            s[~mask] = -np.inf
            mx = s.max(-1)
            lse[b, h] = mx + np.log(np.exp(s - mx[:, None]).sum(-1))
            dq, dk, dv = OM.attention_bwd(dy[b, :, h * hd:(h + 1) * hd].astype(np.float64), q, k, v, p)
            dqkv[b, :, h * hd:(h + 1) * hd] = dq
            dqkv[b, :, C + j * hd:C + (j + 1) * hd] += dk
            dqkv[b, :, C + Ckv + j * hd:C + Ckv + (j + 1) * hd] += dv
    return y, lse, dqkv


def _segments(g, B, T, E, seed):
    s = synthetic.token_stream(B * T, seed=seed, vocab=E, eot=E, mean_doc=90)
    x = s.reshape(B, T).astype(np.int32)
    x[0, [t for t in (0, 64, 129) if t < T]] = E
    return x, g.op_segment_starts(dev(x), E)


@pytest.mark.parametrize("B,T,H,Hkv,doc", [(2, 300, 6, 2, False), (1, 1024, 4, 1, False), (2, 257, 6, 3, True),
                                           (1, 128, 2, 2, True)])
def test_attention_bf16_gqa_vs_oracle(g, B, T, H, Hkv, doc):
    import torch
    hd = 64
    announce(f"attention bf16 gqa B={B} T={T} H={H} Hkv={Hkv} doc={doc}")
    rng = np.random.default_rng(T + H + Hkv)
    W = (H + 2 * Hkv) * hd
    qkv = bf16_round(rng.standard_normal((B * T, W)).astype(np.float32))
    dy = bf16_round(rng.standard_normal((B * T, H * hd)).astype(np.float32))
    masks, seg = None, None
    if doc:
        x, seg = _segments(g, B, T, 400, seed=T)
        masks, _ = OM.packed_rows(x, 400)
    y_ref, lse_ref, dqkv_ref = _oracle(qkv, B, T, H, Hkv, hd, dy.reshape(B, T, -1), masks)
    dq = dev(qkv, torch.bfloat16)
    y = torch.zeros((B * T, H * hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dq, y, lse, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    yh = host(y).reshape(B, T, -1)
    assert cosine(yh, y_ref) > 0.9999
    assert np.abs(yh - y_ref).max() <= 2e-2 * max(1.0, np.abs(y_ref).max())
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-4, atol=1e-3)
    dqkv = torch.zeros((B * T, W), dtype=torch.bfloat16, device="cuda")
    g.op_attention_bwd(dq, y, dev(dy, torch.bfloat16), lse, dqkv, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    got = host(dqkv).reshape(B, T, -1)
    C, Ckv = H * hd, Hkv * hd
    for name, sl in (("dq", slice(0, C)), ("dk", slice(C, C + Ckv)), ("dv", slice(C + Ckv, W))):
        assert cosine(got[..., sl], dqkv_ref[..., sl]) > 0.999, name
        assert np.abs(got[..., sl] - dqkv_ref[..., sl]).max() <= 3e-2 * max(1.0, np.abs(dqkv_ref[..., sl]).max()), name


@pytest.mark.parametrize("doc", [False, True])
def test_attention_fp32_gqa_vs_oracle(g, doc):
    import torch
    B, T, H, Hkv, hd = 2, 70, 4, 2, 16
    announce(f"attention fp32 gqa doc={doc}")
    rng = np.random.default_rng(5)
    W = (H + 2 * Hkv) * hd
    qkv = rng.standard_normal((B * T, W)).astype(np.float32)
    dy = rng.standard_normal((B * T, H * hd)).astype(np.float32)
    masks, seg = None, None
    if doc:
        x, seg = _segments(g, B, T, 50, seed=3)
        masks, _ = OM.packed_rows(x, 50)
    y_ref, lse_ref, dqkv_ref = _oracle(qkv, B, T, H, Hkv, hd, dy.reshape(B, T, -1), masks)
    y = torch.zeros((B * T, H * hd), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    g.op_attention_fwd(dev(qkv), y, lse, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    np.testing.assert_allclose(host(y).reshape(B, T, -1), y_ref, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(host(lse), lse_ref, rtol=1e-5, atol=1e-5)
    dqkv = torch.zeros((B * T, W), dtype=torch.float32, device="cuda")
    g.op_attention_bwd(dev(qkv), y, dev(dy), lse, dqkv, B, T, H, hd, seg=seg, n_kv_head=Hkv)
    np.testing.assert_allclose(host(dqkv).reshape(B, T, -1), dqkv_ref, rtol=1e-4, atol=1e-4)


def test_attention_gqa_rejects_bad_head_counts(g):
    import torch
    announce("attention gqa argument checks")
    qkv = torch.zeros((64, 7 * 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((64, 4 * 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
    for bad in (3, 0, -1):
        with pytest.raises(g.GPT2Error) as e:
            g.op_attention_fwd(qkv, y, lse, 1, 64, 4, 64, n_kv_head=bad)
        assert e.value.status == g._ffi.GPT2_ERR_SHAPE


SMALL_ROT = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=4, n_embd=256, mlp_hidden=160)


def _rotary_parity(g, cfg, B, T, seed, eot=None, mean_doc=1000.0):
    oc = OMM.ModernConfig(cfg.vocab_size, cfg.block_size, cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.mlp_hidden,
                          n_kv_head=cfg.n_kv_head)
    m = g.GPT2(cfg)
    params = synthetic.random_params(OMM.param_specs(oc), seed=seed)
    load_params(m, params)
    m.zero_grad()
    if eot is not None:
        m.set_doc_mask(eot)
    V = cfg.vocab_size if eot is None else eot
    s = synthetic.token_stream(B * T + 1, seed=seed, vocab=V, eot=V if eot is not None else synthetic.EOT_ID,
                               mean_doc=mean_doc)
    s = np.where(s < cfg.vocab_size, s, s % cfg.vocab_size).astype(np.int32)
    x, y = synthetic.micro_batch(s, 0, B, T)
    import torch
    tl = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    loss = m.fwd_bwd(dev(x), dev(y), loss_scale=0.5, token_loss=tl)
    assert m.status() == 0
    grads = read_named(m, m.grads)
    m.close()
    lref, rl, gref = OMM.fwd_bwd(oc, params, x, y, scale=0.5, eot=eot)
    return float(host(loss)[0]), host(tl), lref, rl, grads, gref


@pytest.mark.parametrize("Hkv,doc", [(2, False), (1, False), (2, True)])
def test_rotary_small_gqa_step_parity(g, Hkv, doc):
    cfg = g.ModelConfig(**SMALL_ROT, max_batch=3, precision=g.PRECISION_BF16, arch=g.ARCH_ROTARY, n_kv_head=Hkv)
    announce(f"rotary small gqa Hkv={Hkv} doc={doc} fwd_bwd B=3 T=200")
    loss, tl, lref, rl, grads, gref = _rotary_parity(g, cfg, 3, 200, 31, eot=1023 if doc else None, mean_doc=50)
    assert abs(loss - lref) / abs(lref) <= 1e-2
    assert np.abs(tl.reshape(-1) - rl).max() <= 0.05
    for k in gref:
        if np.linalg.norm(gref[k]) > 0:
            c = cosine(grads[k], gref[k])
            assert c >= 0.999, (k, c)


@pytest.mark.timeout(600)
def test_rotary_124m_gqa_step_parity_b1(g):
    """The rotary variant at its real width with 12 query heads sharing 4
    key/value heads, one sequence of 1024 tokens: loss and every gradient
    tensor against the float32 oracle."""
    cfg = g.ModelConfig(50304, 1024, 12, 12, 768, 2048, 1, g.PRECISION_BF16, g.ARCH_ROTARY, n_kv_head=4)
    announce("rotary 124m gqa (12 q / 4 kv heads) fwd_bwd B=1 T=1024")
    loss, tl, lref, rl, grads, gref = _rotary_parity(g, cfg, 1, 1024, 42)
    assert abs(loss - lref) / abs(lref) <= 1e-2
    worst = min((cosine(grads[k], gref[k]), k) for k in gref if np.linalg.norm(gref[k]) > 0)
    assert worst[0] >= 0.999, worst
