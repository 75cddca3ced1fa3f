"""The training loop around the step and the HIP graph of a micro-step, on
the GPU, through the C-ABI.

* A captured micro-step replayed over fresh token buffers gives the eager
  step's loss and gradients (eager work and synchronisations between the
  replays; every replay checked).
* The loop (warmed-up cosine schedule, accumulation, clip + AdamW, one
  readback per step) follows the oracle loop step by step in float32 mode.
* In bf16 mode the loop, with graph replays, overfits one fixed batch.
"""

import math

import numpy as np
import pytest

from gpu_util import announce, dev, host, load_params, read_named
from oracle import model as OM
import oracle
import synthetic

pytestmark = pytest.mark.gpu

SMALL_BF16 = dict(vocab_size=1024, block_size=256, n_layer=2, n_head=2, n_embd=128, mlp_hidden=512)


@pytest.fixture(scope="module")
def g():
    import torch
    import gpt_pretraining_step_amd as g
    assert torch.cuda.is_available()
    g.lib()
    return g


def ocfg(c):
    return OM.Config(c.vocab_size, c.block_size, c.n_layer, c.n_head, c.n_embd, c.mlp_hidden)


def test_graph_replay_matches_eager(g):
    import torch
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=2, precision=g.PRECISION_BF16)
    announce("graph replay vs eager, small bf16 B=2 T=128")
    m = g.GPT2(cfg)
    load_params(m, synthetic.random_params(OM.param_specs(ocfg(cfg)), seed=8))
    rng = np.random.default_rng(1)
    batches = [(rng.integers(0, cfg.vocab_size, size=(2, 128)).astype(np.int32),
                rng.integers(0, cfg.vocab_size, size=(2, 128)).astype(np.int32)) for _ in range(4)]
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ref = []
    for x, y in batches:
        m.zero_grad()
        m.fwd_bwd(dev(x), dev(y), loss_scale=0.5, loss_out=loss)
        ref.append((float(host(loss)[0]), host(m.grads).copy()))
    tok = dev(batches[0][0])
    tgt = dev(batches[0][1])
    m.graph_capture(tok, tgt, loss_scale=0.5, loss_out=loss)
    for k, (x, y) in enumerate(batches):
        # eager work of the program's own between the replays
        m.zero_grad()
        m.fwd_bwd(dev(batches[-1 - k][0]), dev(batches[-1 - k][1]), loss_scale=0.5)
        torch.cuda.synchronize()
        m.zero_grad()
        tok.copy_(torch.from_numpy(x).cuda())
        tgt.copy_(torch.from_numpy(y).cuda())
        m.graph_launch()
        torch.cuda.synchronize()
        assert m.status() == 0
        got_loss, got_grads = float(host(loss)[0]), host(m.grads)
        assert got_loss == pytest.approx(ref[k][0], rel=1e-6), k
        np.testing.assert_allclose(got_grads, ref[k][1], rtol=1e-5, atol=1e-7, err_msg=f"replay {k}")
    # a second replay without zeroing adds the same gradients again
    m.graph_launch()
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(m.grads), 2 * ref[-1][1], rtol=1e-5, atol=1e-7)
    m.close()


def test_graph_capture_rejections(g):
    import torch
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=2, precision=g.PRECISION_BF16)
    m = g.GPT2(cfg)
    with pytest.raises(g.GPT2Error):
        m.graph_launch()  # nothing captured yet
    x = dev(np.zeros((2, 64), dtype=np.int32))
    m.profile(True)
    with pytest.raises(g.GPT2Error):
        m.graph_capture(x, x)  # not while profiling
    m.profile(False)
    m.close()


def test_loop_follows_the_oracle_loop_fp32(g):
    """Five optimizer steps of two micro-batches each, warmup 2 of 5 steps:
    per-step loss, pre-clip norm and learning rate against the oracle loop."""
    cfg = g.TINY_CHAR_FP32
    oc = ocfg(cfg)
    announce("fp32 loop vs oracle loop, 5 steps")
    params = synthetic.random_params(OM.param_specs(oc), seed=12)
    m = g.GPT2(cfg)
    load_params(m, params)
    stream = synthetic.uniform_stream(20 * 4 * 64 + 1, 66, seed=7)
    mb = [synthetic.micro_batch(stream, k, 4, 64) for k in range(10)]
    sched = g.train.Schedule(max_lr=3e-3, min_lr=3e-4, warmup=2, max_steps=5)
    hist = g.train.train(m, lambda s: [(dev(x.astype(np.int32)), dev(y.astype(np.int32))) for x, y in mb[2 * s:2 * s + 2]],
                         5, sched, weight_decay=0.1)
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    ref = oracle.train(oc, p64, lambda s: mb[2 * s:2 * s + 2], 5, OM.fwd_bwd, 3e-3, 3e-4, 2, 5, weight_decay=0.1)
    for s, ((l, n, lr), (lr_, nr, lrr)) in enumerate(zip(hist, ref)):
        assert lr == pytest.approx(lrr, rel=1e-6), s
        assert l == pytest.approx(lr_, rel=1e-3), s
        assert n == pytest.approx(nr, rel=1e-2), s
    got = read_named(m, m.params)
    worst = max(float(np.abs(got[k] - p64[k]).max()) for k in p64)
    assert worst <= 1e-3, worst
    m.close()


def test_loop_overfits_a_fixed_batch_bf16_with_graphs(g):
    cfg = g.ModelConfig(**SMALL_BF16, max_batch=4, precision=g.PRECISION_BF16)
    announce("bf16 loop with graph replays, 30 steps on one batch")
    m = g.GPT2(cfg)
    m.init_params(seed=42)
    stream = synthetic.token_stream(4 * 128 + 1, seed=5)
    stream = np.where(stream < cfg.vocab_size, stream, stream % cfg.vocab_size).astype(np.int32)
    x, y = synthetic.micro_batch(stream, 0, 4, 128)
    xd, yd = dev(x), dev(y)
    sched = g.train.Schedule(max_lr=3e-3, min_lr=3e-4, warmup=5, max_steps=30)
    hist = g.train.train(m, lambda s: [(xd, yd), (xd, yd)], 30, sched, weight_decay=0.0, graph=True)
    assert hist[0][0] == pytest.approx(math.log(cfg.vocab_size), abs=0.3)
    assert all(math.isfinite(h[0]) and math.isfinite(h[1]) for h in hist)
    assert hist[-1][0] < 0.5 * hist[0][0], [round(h[0], 3) for h in hist]
    assert [h[2] for h in hist[:5]] == pytest.approx([3e-3 * (s + 1) / 5 for s in range(5)])
    m.close()
