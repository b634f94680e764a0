"""Seeded generators for the workloads of the ternary-weight GEMM.

Distributions follow the workloads the pages benchmark on (layer shapes of
LLaMA-style ternary models) as written out in the project's workload table:

* activations X: fp32 standard normal, cast to fp16 (round to nearest even);
* latent weights W: fp32 normal with standard deviation ``sigma`` (0.02);
* ternary weights drawn directly: i.i.d. with P(0) = p and P(+1) = P(-1);
* per-256-block fp16 scales: fp32 uniform on [lo, hi), cast to fp16.

Every generator takes an explicit ``numpy.random.Generator``; ``seed_for``
derives one from a (config, tensor, layer) tuple so that every array of a
workload can be regenerated on its own.
"""

from __future__ import annotations

import numpy as np

#: Number of weights that share one fp16 scale along K.
BLOCK = 256


def seed_for(*key: int) -> np.random.Generator:
    """A generator whose stream depends only on the integer tuple ``key``."""
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def activations_fp16(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """X[M][K] fp16 from a standard normal drawn in fp32."""
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def latent_weights_f32(rng: np.random.Generator, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """Latent W[N][K] fp32 from N(0, sigma^2)."""
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def ternary_iid(rng: np.random.Generator, N: int, K: int, p_zero: float) -> np.ndarray:
    """T[N][K] int8 in {-1, 0, 1}: zero with probability p_zero, else +-1 equally likely."""
    out = np.empty((N, K), dtype=np.int8)
    rows = max(1, (1 << 22) // max(K, 1))  # draw in slabs to bound peak memory
    half = np.float32(p_zero + (1.0 - p_zero) / 2.0)
    pz = np.float32(p_zero)
    for r0 in range(0, N, rows):
        r1 = min(N, r0 + rows)
        u = rng.random((r1 - r0, K), dtype=np.float32)
        slab = np.where(u < pz, 0, np.where(u < half, 1, -1))
        out[r0:r1] = slab.astype(np.int8)
    return out


def block_scales_fp16(rng: np.random.Generator, N: int, K: int,
                      lo: float = 0.01, hi: float = 0.03) -> np.ndarray:
    """scales[N][K/256] fp16 from U(lo, hi) drawn in fp32."""
    nb = K // BLOCK
    s = rng.uniform(lo, hi, size=(N, nb)).astype(np.float32)
    return s.astype(np.float16)
