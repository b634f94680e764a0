"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import functools

import numpy as np

from oracle import dequantize_ref, gemm_ref
from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid

#: Acceptance bound of the product: max|Y - Y_ref| <= REL_TOL * max|Y_ref|.
REL_TOL = 4e-3


def check_close(Y, Yref, label=""):
    """Y (fp16, any array-like) against the fp64 oracle; returns the error in
    units of max|Y_ref| and of fp16 ulps of |Y_ref| for logging."""
    Y64 = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    assert Y64.shape == Yref.shape, (label, Y64.shape, Yref.shape)
    assert np.all(np.isfinite(Y64)), label
    big = float(np.max(np.abs(Yref))) if Yref.size else 0.0
    err = float(np.max(np.abs(Y64 - Yref))) if Yref.size else 0.0
    if big == 0.0:
        assert err == 0.0, (label, err)
        return 0.0, 0.0
    ulp = np.spacing(np.abs(Yref).astype(np.float16)).astype(np.float64)
    ulp_err = float(np.max(np.abs(Y64 - Yref) / np.maximum(ulp, 2.0 ** -24)))
    assert err <= REL_TOL * big, f"{label}: max err {err:.3e} > {REL_TOL} * {big:.3e} (ulps {ulp_err:.1f})"
    return err / big, ulp_err


@functools.lru_cache(maxsize=8)
def iid_problem(N, K, p_zero, seed):
    """Ternary weights i.i.d. and U(0.01, 0.03) block scales (numpy, host)."""
    rng = seed_for(seed, N, K, int(p_zero * 1000))
    T = ternary_iid(rng, N, K, p_zero)
    s = block_scales_fp16(rng, N, K)
    return T, s


def activations(M, K, seed):
    return activations_fp16(seed_for(seed, M, K, 99), M, K)


def ref(X, T, s, cols=None):
    return gemm_ref(X, T, s, cols=cols)


class DenseRef:
    """The oracle's product for one (T, s) and several X: ``dequantize_ref``
    once, then ``X64 @ Wd.T`` per call, the same arithmetic as ``gemm_ref``
    without rebuilding the fp64 matrix (1.9 GB at 28672 x 8192) every time."""

    def __init__(self, T, s):
        self.WdT = dequantize_ref(T, s).T

    def __call__(self, X, cols=None):
        W = self.WdT if cols is None else self.WdT[:, np.asarray(cols)]
        return np.asarray(X).astype(np.float64) @ W


def strat_cols(N, seed, group=16, edge=32):
    """Columns for a sampled check of a wide output: one random column in every
    ``group`` consecutive columns, plus the first and last column of every
    ``edge``-column tile (so both edges of every 32-, 64- and 128-wide weight
    tile and every row group of 16), sorted and unique."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, N, group)
    pick = starts + rng.integers(0, group, size=starts.size)
    tiles = np.arange(0, N, edge)
    cols = np.concatenate([pick, tiles, np.minimum(tiles + edge - 1, N - 1), [N - 1]])
    return np.unique(cols[cols < N])
