"""The seeded input generators: the stand-in token stream has the shape the
pages' data has (EOT before every document, consecutive windows shifted by
one, Zipf ids), and the batches keep the continuity the pages point out."""

import numpy as np

import synthetic


def test_micro_batches_shift_and_continuity():
    # Zero to Frontier, GPT chapter, "In PyTorch": the last target of one
    # batch is the first input of the next.
    s = synthetic.token_stream(3 * 4 * 16 + 1, seed=3)
    x0, y0 = synthetic.micro_batch(s, 0, 4, 16)
    x1, y1 = synthetic.micro_batch(s, 1, 4, 16)
    assert np.array_equal(x0.reshape(-1)[1:], y0.reshape(-1)[:-1])
    assert y0.reshape(-1)[-1] == x1.reshape(-1)[0]
    assert x0.dtype == np.int32 and x0.shape == (4, 16)


def test_stream_statistics():
    n = 400_000
    s = synthetic.token_stream(n)
    assert s.min() >= 0 and s.max() < 50257
    eot = np.flatnonzero(s == synthetic.EOT_ID)
    assert eot[0] == 0
    # one EOT per ~1000 tokens (plus Zipf draws that land on the EOT id)
    gaps = np.diff(eot)
    assert 800 < np.median(gaps) < 1200 or 700 < gaps.mean() < 1100
    # top Zipf(1.1) rank carries ~13.9% of the ids
    counts = np.bincount(s, minlength=50257)
    top = np.sort(counts)[::-1]
    assert abs(top[0] / n - 0.139) < 0.01
    assert abs(top[:5].sum() / n - 0.299) < 0.015


def test_lmhead_inputs_shape_and_ignore_count():
    h, w, t = synthetic.lmhead_inputs(M=2048, C=64, V=50304)
    assert h.shape == (2048, 64) and w.shape == (50304, 64)
    assert int((t == -1).sum()) == round(0.1 * 2048)
    assert t.max() < 50257
    # values are exactly representable in bfloat16
    assert np.all((h.view(np.uint32) & 0xFFFF) == 0)
    assert np.all((w.view(np.uint32) & 0xFFFF) == 0)


def test_round_to_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.3], dtype=np.float32)
    r = synthetic.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                    # tie -> even mantissa
    assert r[2] == 1.0 + 4 * 2 ** -8      # tie -> even mantissa (rounds up)
    assert r[3] == -2.5
    assert abs(r[4] - 3.3) < 3.3 * 2 ** -8
