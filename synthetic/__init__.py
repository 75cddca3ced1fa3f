"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input generation only: token streams, batches cut from them,
random tensors of caller-given shapes.  It contains none of the model's
arithmetic, imports neither the oracle nor the HIP binding, and both sides
receive exactly the arrays produced here.

Stand-ins (the pages train on FineWeb-Edu GPT-2 token shards, which are not
available): a token stream whose ids follow a Zipf law (exponent 1.1) over a
seeded permutation of the 50257 GPT-2 ids, cut into documents of length
1 + Geometric(1/1000), each preceded by the end-of-text id 50256 (the pages put
the separator before every document).  Micro-batches are consecutive windows
of B*T + 1 tokens with targets shifted by one, so the last target of one batch
is the first input of the next.
"""

from __future__ import annotations

import numpy as np

GPT2_VOCAB = 50257
EOT_ID = 50256
DATA_SEED = 1337
PARAM_SEED = 42


def zipf_probs(n: int = GPT2_VOCAB, s: float = 1.1) -> np.ndarray:
    ranks = np.arange(1, n + 1, dtype=np.float64)
    w = ranks ** (-s)
    return w / w.sum()


def zipf_ids(rng: np.random.Generator, count: int, n: int = GPT2_VOCAB, s: float = 1.1,
             perm: np.ndarray | None = None) -> np.ndarray:
    """``count`` ids drawn by inverse CDF from a Zipf(s) law over ranks 1..n,
    mapped to ids through ``perm`` (rank r -> perm[r-1])."""
    cdf = np.cumsum(zipf_probs(n, s))
    cdf[-1] = 1.0
    u = rng.random(count)
    rank0 = np.searchsorted(cdf, u, side="right")
    rank0 = np.minimum(rank0, n - 1)
    if perm is None:
        return rank0.astype(np.int64)
    return perm[rank0].astype(np.int64)


def token_stream(n_tokens: int, seed: int = DATA_SEED, vocab: int = GPT2_VOCAB, eot: int = EOT_ID,
                 s: float = 1.1, mean_doc: float = 1000.0) -> np.ndarray:
    """int32 stream of ``n_tokens`` ids: documents of Zipf ids, each preceded
    by ``eot``; document lengths 1 + Geometric(1/mean_doc)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(vocab)
    out = np.empty(n_tokens, dtype=np.int32)
    pos = 0
    while pos < n_tokens:
        out[pos] = eot
        pos += 1
        length = 1 + int(rng.geometric(1.0 / mean_doc))
        take = min(length, n_tokens - pos)
        if take > 0:
            out[pos:pos + take] = zipf_ids(rng, take, vocab, s, perm)
            pos += take
    return out


def uniform_stream(n_tokens: int, vocab: int, seed: int = DATA_SEED) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=n_tokens).astype(np.int32)


def micro_batch(stream: np.ndarray, k: int, B: int, T: int):
    """Micro-batch k: window stream[k*B*T : k*B*T + B*T + 1]; x = window[:-1],
    y = window[1:], both viewed as [B, T] (int32)."""
    start = k * B * T
    buf = stream[start:start + B * T + 1]
    if buf.size != B * T + 1:
        raise ValueError("stream too short for micro-batch %d" % k)
    return buf[:-1].reshape(B, T).copy(), buf[1:].reshape(B, T).copy()


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned
    as float32, so both sides can hold the exact same numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    r = ((bits + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def lmhead_inputs(M: int = 65536, C: int = 768, V: int = 50304, ignore_frac: float = 0.1,
                  seed: int = DATA_SEED):
    """Inputs of the isolated lm_head + cross-entropy workload: hidden [M, C]
    ~ N(0, 1), weight [V, C] ~ N(0, 0.02^2), both rounded to bf16 values;
    targets Zipf over the GPT-2 ids with exactly round(ignore_frac * M)
    positions set to -1."""
    rng = np.random.default_rng(seed)
    hidden = round_to_bf16(rng.standard_normal((M, C), dtype=np.float32))
    weight = round_to_bf16((0.02 * rng.standard_normal((V, C))).astype(np.float32))
    perm = rng.permutation(GPT2_VOCAB)
    targets = zipf_ids(rng, M, GPT2_VOCAB, 1.1, perm).astype(np.int32)
    n_ign = int(round(ignore_frac * M))
    if n_ign > 0:
        targets[rng.choice(M, size=n_ign, replace=False)] = -1
    return hidden, weight, targets


def random_params(specs, seed: int = PARAM_SEED, matrix_std: float = 0.02, vector_std: float = 0.05):
    """Random float32 tensors for the given (name, shape) list: matrices
    ~ N(0, matrix_std^2); vectors whose name contains 'ln_' and ends in
    'weight' ~ 1 + N(0, vector_std^2); other vectors ~ N(0, vector_std^2).
    Used by parity tests so that biases and norm gains are exercised."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in specs:
        z = rng.standard_normal(shape, dtype=np.float32)
        if len(shape) >= 2:
            out[name] = np.float32(matrix_std) * z
        elif "ln_" in name and name.endswith("weight"):
            out[name] = np.float32(1.0) + np.float32(vector_std) * z
        else:
            out[name] = np.float32(vector_std) * z
    return out
