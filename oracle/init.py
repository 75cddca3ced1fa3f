"""Oracle parameter initialisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The init spec is [train-124M] §7 (and the same code on [repro-124M]):
  * every nn.Linear weight and both embeddings ~ N(0, 0.02);
  * the two residual projections (attn.c_proj and mlp.c_proj) use
    std 0.02 * (2 * n_layer) ** -0.5;
  * Linear biases are zero; LayerNorm weight 1 and bias 0 (nn.LayerNorm
    defaults).

The page draws with torch's generator, which nothing here can reproduce.
Both this oracle and the device code instead implement one counter-based
generator from its published definition: Philox4x32-10 (Salmon, Moraes,
Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), turned
into normals by the Box-Muller transform.  The stream is defined as:

  element j of parameter tensor number k (its position in the parameter
  table), under a 64-bit seed s:
    counter = (j // 4 low 32 bits, j // 4 high 32 bits, k, 0x6770 (ascii "gp"))
    key     = (s low 32 bits, s high 32 bits)
    (w0, w1, w2, w3) = philox4x32_10(counter, key)
    u(w) = (w + 0.5) / 2**32                  (in (0, 1))
    r0 = sqrt(-2 ln u(w0)),  r1 = sqrt(-2 ln u(w2))
    z  = (r0 cos 2 pi u(w1), r0 sin 2 pi u(w1), r1 cos 2 pi u(w3), r1 sin 2 pi u(w3))
    value = std_k * z[j % 4]
"""

from __future__ import annotations

import numpy as np

from .model import Config, param_specs

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
STREAM_TAG = 0x6770
MASK32 = 0xFFFFFFFF


def _mulhilo(a, b):
    prod = a.astype(np.uint64) * np.uint64(b)
    return (prod >> np.uint64(32)).astype(np.uint64), (prod & np.uint64(MASK32)).astype(np.uint64)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of 32-bit counters (as uint64
    arrays holding 32-bit values).  Each round: multiply counter words 0 and
    2 by the two Philox multipliers, take high and low halves, mix with the
    odd words and the key; the key is bumped by the Weyl constants between
    rounds."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = np.uint64(k0)
    k1 = np.uint64(k1)
    m32 = np.uint64(MASK32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & m32
            k1 = (k1 + np.uint64(PHILOX_W1)) & m32
        hi0, lo0 = _mulhilo(c0, PHILOX_M0)
        hi1, lo1 = _mulhilo(c2, PHILOX_M1)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & m32, lo1, (hi0 ^ c3 ^ k1) & m32, lo0
    return c0, c1, c2, c3


def normal_from_philox(n: int, tensor_index: int, seed: int) -> np.ndarray:
    """The first n standard normals of tensor ``tensor_index`` (float64)."""
    if n == 0:
        return np.zeros(0)
    calls = (n + 3) // 4
    c = np.arange(calls, dtype=np.uint64)
    w0, w1, w2, w3 = philox4x32_10(c & np.uint64(MASK32), c >> np.uint64(32),
                                   np.full(calls, tensor_index, dtype=np.uint64),
                                   np.full(calls, STREAM_TAG, dtype=np.uint64),
                                   seed & MASK32, (seed >> 32) & MASK32)

    def unif(w):
        return (w.astype(np.float64) + 0.5) / 4294967296.0

    r_a = np.sqrt(-2.0 * np.log(unif(w0)))
    r_b = np.sqrt(-2.0 * np.log(unif(w2)))
    th_a = 2.0 * np.pi * unif(w1)
    th_b = 2.0 * np.pi * unif(w3)
    z = np.empty((calls, 4))
    z[:, 0] = r_a * np.cos(th_a)
    z[:, 1] = r_a * np.sin(th_a)
    z[:, 2] = r_b * np.cos(th_b)
    z[:, 3] = r_b * np.sin(th_b)
    return z.reshape(-1)[:n]


def init_std(cfg: Config, name: str) -> float:
    """std of the normal init of a weight tensor ([train-124M] §7)."""
    if name.endswith("c_proj.weight"):
        return 0.02 * (2 * cfg.n_layer) ** -0.5
    return 0.02


def init_params(cfg: Config, seed: int, dtype=np.float32):
    """All parameters per the init spec, drawn from the Philox stream above."""
    params = {}
    for k, (name, shape) in enumerate(param_specs(cfg)):
        n = int(np.prod(shape))
        if len(shape) >= 2:
            params[name] = (init_std(cfg, name) * normal_from_philox(n, k, seed)).reshape(shape).astype(dtype)
        elif name.endswith("ln_1.weight") or name.endswith("ln_2.weight") or name.endswith("ln_f.weight"):
            params[name] = np.ones(shape, dtype=dtype)
        else:
            params[name] = np.zeros(shape, dtype=dtype)
    return params
