"""fp64 reference for Y = X (gamma * T)^T with T ternary, and for the two packings.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the library.  It shares no
code, table or constant generator with the HIP/C++ path.

Sources (project page "Scaling Laws and Efficient Inference for Ternary Language
Models", unless said otherwise):

* "The model", steps 1-3: gamma = eps + mean|W|, T = round(clip(W/gamma, -1, 1)),
  Y = X (gamma T)^T.  The Spectra project page ("Architecture of TriLM and
  FloatLM") says the same in words: one absolute-mean scale per matrix, each
  weight rounded to the nearest ternary state.
* "Packing ternary weights": d' = d + 1; "2 bits per weight": field j of a byte
  is (b >> 2j) & 3; "1.6 bits per weight": five digits read as a base-3 number
  N in [0, 242], stored as b = floor((256 N + 242) / 243); decoded either by the
  inverse formula (division and modulo) or by multiplying by 3 five times and
  splitting high byte from low byte.
* "Fast inference on CPUs": the 2-bit format carries one 16-bit scale per block
  of 256 weights.
* "TriRun: ternary inference on GPUs": FP16 outputs after FP32 accumulation.

Readings where the pages are silent (each also listed in the design notes):
round() ties go to even; gamma is an exactly rounded fp64 sum over the whole
matrix divided by N*K, plus eps; weight k = 4i + j of a row sits in byte i,
bits 2j..2j+1; in TQ1 the first of five weights is the most significant base-3
digit (the worked example decodes (1, -1, 0, 0, 1) to 2, 0, 1, 1, 2 in weight
order); TQ1 groups never cross rows, the last group of a row is padded with
zero trits, rows are ``ldq`` bytes apart and the bytes past the last group are
zero; both packings take the same fp16 scale table scales[N][K/256]; when
packing from latents every block scale is fp16(gamma), one round-to-nearest-
even step from fp64.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against printed values, closed forms, brute force or textbook special cases;
none is "parity unpinned".
"""

from __future__ import annotations

import math
import struct

import numpy as np

#: Weights per fp16 scale along K ("Fast inference on CPUs": 256-weight blocks).
BLOCK = 256

_POW3 = (81, 27, 9, 3, 1)  # place values of digits 0..4; digit 0 most significant


# --------------------------------------------------------------------------
# Ternarization ("The model", steps 1-2)
# --------------------------------------------------------------------------

def ternarize_ref(W, eps: float):
    """Return (T int8[N][K], gamma) with gamma = eps + mean|W| over the whole matrix.

    The mean is an exactly rounded fp64 sum (``math.fsum``) divided by the
    element count; the decision for each weight is taken on the fp64 quotient
    W / gamma, clipped to [-1, 1] and rounded half to even.
    """
    W64 = np.asarray(W).astype(np.float64)
    if W64.ndim != 2:
        raise ValueError("W must be 2-D [N][K]")
    if not np.all(np.isfinite(W64)):
        raise ValueError("non-finite latent weight")
    count = W64.size
    if count == 0:
        raise ValueError("empty matrix")
    total = math.fsum(np.abs(W64).ravel())
    gamma = float(eps) + total / count
    if not (math.isfinite(gamma) and gamma > 0.0):
        raise ValueError("gamma must be finite and positive")
    q = np.clip(W64 / gamma, -1.0, 1.0)
    T = np.rint(q).astype(np.int8)
    return T, gamma


def fp16_bits_ref(x: float) -> int:
    """IEEE binary16 bit pattern of fp64 ``x``, rounded to nearest even in one step.

    Magnitudes that round past the largest finite half (65504) become infinity.
    """
    try:
        return struct.unpack("<H", struct.pack("<e", float(x)))[0]
    except OverflowError:
        return 0xFC00 if x < 0 else 0x7C00


# --------------------------------------------------------------------------
# 2 bits per weight ("Packing ternary weights" / "2 bits per weight")
# --------------------------------------------------------------------------

def _check_ternary(T):
    T = np.asarray(T)
    if T.ndim != 2:
        raise ValueError("T must be 2-D [N][K]")
    if not np.all((T >= -1) & (T <= 1)):
        raise ValueError("trit outside {-1, 0, 1}")
    return T.astype(np.int64)


def pack_tq2_ref(T) -> np.ndarray:
    """qs[N][K/4]: byte i of a row holds d'(4i + j) in bits 2j..2j+1."""
    T = _check_ternary(T)
    N, K = T.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    d = (T + 1).reshape(N, K // 4, 4)
    qs = d[:, :, 0] | (d[:, :, 1] << 2) | (d[:, :, 2] << 4) | (d[:, :, 3] << 6)
    return qs.astype(np.uint8)


def unpack_tq2_ref(qs, K: int) -> np.ndarray:
    """Inverse of ``pack_tq2_ref``: d' = (b >> 2j) & 3, d = d' - 1; a field of 3 is invalid."""
    qs = np.asarray(qs, dtype=np.uint8)
    N = qs.shape[0]
    if qs.shape[1] != K // 4 or K % 4:
        raise ValueError("qs does not match K")
    b = qs.astype(np.int64)
    fields = np.stack([(b >> (2 * j)) & 3 for j in range(4)], axis=-1)
    if np.any(fields == 3):
        raise ValueError("invalid 2-bit field (3)")
    return (fields - 1).reshape(N, K).astype(np.int8)


# --------------------------------------------------------------------------
# 1.6 bits per weight ("Packing ternary weights" / "1.6 bits per weight")
# --------------------------------------------------------------------------

def tq1_ldq_ref(K: int) -> int:
    """Default row stride in bytes: ceil(K/5) rounded up to a multiple of 16."""
    groups = -(-K // 5)
    return -(-groups // 16) * 16


def tq1_encode_group_ref(digits) -> int:
    """Five shifted digits d' (first weight first) -> stored byte.

    N is their base-3 value with the first digit most significant, and the byte
    is b = floor((N * 2^8 + 242) / 243).
    """
    n = 0
    for dig in digits:
        if dig not in (0, 1, 2):
            raise ValueError("digit outside {0, 1, 2}")
        n = 3 * n + int(dig)
    return (n * 256 + 242) // 243


def tq1_decode_division_ref(b: int):
    """Inverse formula: N = floor(243 b / 256), digits by division and modulo.

    Returns the five digits, or None when b is not the code of any pattern
    (13 of the 256 byte values are unused).
    """
    n = (int(b) * 243) >> 8
    digits = tuple((n // p) % 3 for p in _POW3)
    if tq1_encode_group_ref(digits) != int(b):
        return None
    return digits


def tq1_decode_multiply_ref(b: int):
    """Multiply route: five times, t = 3 q; digit = high byte of t; q = low byte of t."""
    q = int(b)
    out = []
    for _ in range(5):
        t = 3 * q
        out.append(t >> 8)
        q = t & 0xFF
    return tuple(out)


def pack_tq1_ref(T, ldq: int | None = None) -> np.ndarray:
    """qs[N][ldq]: byte g of a row encodes weights 5g..5g+4 (tail padded with d = 0)."""
    T = _check_ternary(T)
    N, K = T.shape
    G = -(-K // 5)
    if ldq is None:
        ldq = tq1_ldq_ref(K)
    if ldq < G:
        raise ValueError("ldq smaller than ceil(K/5)")
    d = np.ones((N, 5 * G), dtype=np.int64)  # d' = 1 is the trit 0
    d[:, :K] = T + 1
    d = d.reshape(N, G, 5)
    n = sum(d[:, :, j] * _POW3[j] for j in range(5))
    b = (n * 256 + 242) // 243
    qs = np.zeros((N, ldq), dtype=np.uint8)
    qs[:, :G] = b.astype(np.uint8)
    return qs


def unpack_tq1_ref(qs, K: int, ldq: int | None = None) -> np.ndarray:
    """Inverse of ``pack_tq1_ref`` by the division route.

    Raises ValueError for an unused byte value or a non-zero padding trit.
    Bytes past the last group of a row are not inspected.
    """
    if ldq is None:
        ldq = tq1_ldq_ref(K)
    qs = np.asarray(qs, dtype=np.uint8)
    N = qs.shape[0]
    G = -(-K // 5)
    if qs.shape[1] != ldq or ldq < G:
        raise ValueError("qs does not match ldq")
    b = qs[:, :G].astype(np.int64)
    n = (b * 243) >> 8
    digits = np.stack([(n // p) % 3 for p in _POW3], axis=-1)  # [N][G][5]
    re = (sum(digits[:, :, j] * _POW3[j] for j in range(5)) * 256 + 242) // 243
    if np.any(re != b):
        raise ValueError("byte is not a valid 1.6-bit code")
    flat = digits.reshape(N, 5 * G)
    if np.any(flat[:, K:] != 1):
        raise ValueError("non-zero padding trit")
    return (flat[:, :K] - 1).astype(np.int8)


# --------------------------------------------------------------------------
# The product ("The model", step 3; FP16 in, FP32 accumulate, FP16 out on GPU)
# --------------------------------------------------------------------------

def dequantize_ref(T, scales) -> np.ndarray:
    """Wd[n][k] = scales[n][k // 256] * T[n][k] in fp64."""
    T = np.asarray(T)
    s = np.asarray(scales).astype(np.float64)
    N, K = T.shape
    if K % BLOCK or s.shape != (N, K // BLOCK):
        raise ValueError("scales must be [N][K/256]")
    return np.repeat(s, BLOCK, axis=1) * T.astype(np.float64)


def gemm_ref(X, T, scales, cols=None) -> np.ndarray:
    """Y_ref = X (s . T)^T in fp64; ``cols`` restricts the output columns n.

    Every product of an fp16 activation, an fp16 scale and a trit is exact in
    fp64, so Y_ref differs from the real-number result only by the rounding of
    a K-term fp64 sum.
    """
    X64 = np.asarray(X).astype(np.float64)
    T = np.asarray(T)
    s = np.asarray(scales)
    if cols is not None:
        cols = np.asarray(cols)
        T = T[cols]
        s = s[cols]
    Wd = dequantize_ref(T, s)
    if X64.shape[1] != Wd.shape[1]:
        raise ValueError("X and T disagree on K")
    return X64 @ Wd.T


def gemm_bruteforce_ref(X, T, scales) -> np.ndarray:
    """Triple loop with an exactly rounded sum per output (tiny shapes only)."""
    X = np.asarray(X).astype(np.float64)
    T = np.asarray(T)
    s = np.asarray(scales).astype(np.float64)
    M, K = X.shape
    N = T.shape[0]
    Y = np.zeros((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            Y[m, n] = math.fsum(float(X[m, k]) * float(s[n, k // BLOCK]) * int(T[n, k])
                                for k in range(K))
    return Y


def silu_ref(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (the gate of the SwiGLU MLP the
    project page's architecture section names)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(X, T_gate, s_gate, T_up, s_up, cols=None) -> np.ndarray:
    """silu(X (s_g . T_g)^T) * (X (s_u . T_u)^T) in fp64: the gated MLP input
    of the decode step, both products as gemm_ref."""
    g = gemm_ref(X, T_gate, s_gate, cols)
    u = gemm_ref(X, T_up, s_up, cols)
    return silu_ref(g) * u


def gemm_bwd_x_ref(dY, T, scales, cols=None) -> np.ndarray:
    """dX = dY (s . T) in fp64: the input gradient of Y = X (s . T)^T (the
    backward pass of quantization-aware training, "The model": the forward
    uses the ternary weights, the backward the same product transposed).
    ``cols`` restricts the output columns k (the same product, fewer columns
    of s . T)."""
    dY64 = np.asarray(dY).astype(np.float64)
    if cols is None:
        Wd = dequantize_ref(T, scales)
    else:
        cols = np.asarray(cols)
        T = np.asarray(T)
        s64 = np.asarray(scales).astype(np.float64)
        Wd = s64[:, cols // 256] * T[:, cols].astype(np.float64)
    if dY64.shape[1] != Wd.shape[0]:
        raise ValueError("dY and T disagree on N")
    return dY64 @ Wd


def ste_grad_w_ref(dY, X, dW_in=None, rows=None) -> np.ndarray:
    """Gradient that reaches the latent weights of one ternary linear, in fp64.

    "The model" (project page) and "Architecture of TriLM and FloatLM" (Spectra
    page): the forward pass uses the effective weights gamma * T, with
    T = round(clip(W / gamma, -1, 1)), and a straight-through estimator carries
    the gradient back to the latent floating-point weights W.  Read plainly,
    the estimator treats the whole quantizer W -> gamma * T as the identity in
    the backward pass, so the latent weights receive exactly the gradient of
    the loss with respect to the effective weights of Y = X (gamma T)^T:

        dW[n][k] = sum_m dY[m][n] * X[m][k]      (dW = dY^T X)

    with gamma not differentiated and no mask outside the clip window (the
    pages name none).  It does not depend on W, gamma or T.  ``dW_in`` (fp32
    or fp64 [N][K]) is added when given: gradient accumulation over
    micro-batches.  ``rows`` restricts the output rows n.
    """
    dY64 = np.asarray(dY).astype(np.float64)
    X64 = np.asarray(X).astype(np.float64)
    if dY64.ndim != 2 or X64.ndim != 2 or dY64.shape[0] != X64.shape[0]:
        raise ValueError("dY [M][N] and X [M][K] must share M")
    if rows is not None:
        dY64 = dY64[:, np.asarray(rows)]
    G = dY64.T @ X64
    if dW_in is not None:
        base = np.asarray(dW_in).astype(np.float64)
        if rows is not None:
            base = base[np.asarray(rows)]
        G = base + G
    return G
