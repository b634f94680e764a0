"""Pins for the fp64 oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a value
printed on the pages (``tests/golden/page_facts.json``), a hand-worked case of
the page's definition, a closed form, brute force on tiny inputs, or a textbook
special case.  The comments say which plausible mistake each one catches.
"""

import json
import math
import os
import struct

import numpy as np
import pytest

from oracle import (
    BLOCK,
    dequantize_ref,
    fp16_bits_ref,
    gemm_bruteforce_ref,
    gemm_ref,
    pack_tq1_ref,
    pack_tq2_ref,
    ternarize_ref,
    tq1_decode_division_ref,
    tq1_decode_multiply_ref,
    tq1_encode_group_ref,
    tq1_ldq_ref,
    unpack_tq1_ref,
    unpack_tq2_ref,
)
from synth import block_scales_fp16, activations_fp16, latent_weights_f32, seed_for, ternary_iid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


@pytest.fixture(scope="module")
def facts():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- TQ1 codec

def test_tq1_worked_example(facts):
    """The page's worked example: (1, -1, 0, 0, 1) decodes to 2, 0, 1, 1, 2.

    Catches a reversed digit order (least significant first would decode to
    2, 1, 1, 0, 2) and a wrong rescale.  By hand: N = 2*81 + 0*27 + 1*9 + 1*3 + 2
    = 176 and b = ceil(176 * 256 / 243) = 186; 186*3 = 558 -> 2 | 46 -> 138 -> 0
    | 138 -> 414 -> 1 | 158 -> 474 -> 1 | 218 -> 654 -> 2.
    """
    ex = facts["tq1_worked_example"]
    w = np.array([ex["weights"]], dtype=np.int8)
    qs = pack_tq1_ref(w)
    b = int(qs[0, 0])
    assert b == 186
    assert list(tq1_decode_multiply_ref(b)) == ex["decoded_shifted_digits"]
    assert list(tq1_decode_division_ref(b)) == ex["decoded_shifted_digits"]
    assert [d - 1 for d in ex["decoded_shifted_digits"]] == ex["weights"]
    assert unpack_tq1_ref(qs, 5).tolist() == [ex["weights"]]


def test_tq1_all_patterns_both_decoders(facts):
    """All 243 five-trit patterns round-trip through both decoders; the code is injective."""
    n_pat = facts["tq1_combinations"]["patterns"]
    assert 3 ** 5 == n_pat and 2 ** 8 == facts["tq1_combinations"]["byte_values"]
    seen = {}
    for n in range(n_pat):
        digits = tuple((n // 3 ** (4 - j)) % 3 for j in range(5))
        b = tq1_encode_group_ref(digits)
        assert 0 <= b <= 255
        assert tq1_decode_multiply_ref(b) == digits
        assert tq1_decode_division_ref(b) == digits
        assert b not in seen
        seen[b] = digits
    assert len(seen) == 243
    # closed-form endpoints: N = 0 -> 0, all-zero trits (N = 121) -> 128, N = 242 -> 255
    assert tq1_encode_group_ref((0, 0, 0, 0, 0)) == 0
    assert tq1_encode_group_ref((1, 1, 1, 1, 1)) == 128
    assert tq1_encode_group_ref((2, 2, 2, 2, 2)) == 255
    unused = sorted(set(range(256)) - set(seen))
    assert unused == [1, 20, 40, 60, 79, 99, 119, 138, 158, 178, 197, 217, 237]
    for b in unused:
        assert tq1_decode_division_ref(b) is None


def test_tq1_multiply_decoder_needs_the_rescale():
    """Storing the raw base-3 value N instead of b breaks the multiply decoder."""
    bad = 0
    for n in range(243):
        digits = tuple((n // 3 ** (4 - j)) % 3 for j in range(5))
        if tq1_decode_multiply_ref(n) != digits:
            bad += 1
    assert bad > 200


def _lossless(k, p):
    """Brute force: b = ceil(N 2^p / 3^k) fits p bits, is injective, and the
    multiply-by-3 decoder with a p-bit split recovers every k-digit pattern."""
    codes = set()
    for n in range(3 ** k):
        b = (n * 2 ** p + 3 ** k - 1) // 3 ** k
        if b >= 2 ** p:
            return False
        codes.add(b)
        q, out = b, []
        for _ in range(k):
            t = 3 * q
            out.append(t >> p)
            q = t & (2 ** p - 1)
        m = 0
        for dig in out:
            if dig > 2:
                return False
            m = 3 * m + dig
        if m != n:
            return False
    return len(codes) == 3 ** k


def test_lossless_iff_condition():
    """k trits in p bits are lossless exactly when 2^p > 3^k (k <= 6, p <= 10)."""
    for k in range(1, 7):
        for p in range(1, 11):
            assert _lossless(k, p) == (2 ** p > 3 ** k), (k, p)
    best = {k: min(p for p in range(1, 80) if 2 ** p > 3 ** k) / k for k in range(1, 7)}
    assert best[5] == 1.6 and best[5] == min(best.values())
    assert [round(best[k], 3) for k in range(1, 7)] == [2.0, 2.0, 1.667, 1.75, 1.6, 1.667]
    # as k grows the best ratio approaches log2(3)
    ratios = [min(p for p in range(1, 400) if 2 ** p > 3 ** k) / k for k in range(1, 200)]
    assert abs(min(ratios[100:]) - math.log2(3)) < 0.01


def test_bits_per_weight(facts):
    blk = facts["tq2_block"]
    # sizes the oracle's TQ2 packing actually produces for one 256-weight block
    T = np.zeros((1, BLOCK), dtype=np.int8)
    code_bytes = pack_tq2_ref(T).nbytes
    assert code_bytes == blk["code_bytes"]
    assert code_bytes + blk["scale_bits"] // 8 == blk["block_bytes"]
    assert (code_bytes * 8 + blk["scale_bits"]) / BLOCK == blk["bits_per_weight"]
    # TQ1: five weights per byte
    assert pack_tq1_ref(np.zeros((1, 5), dtype=np.int8))[0, :1].nbytes * 8 / 5 == facts["tq1_bits_per_weight"]["value"]
    ent = math.log2(3)
    assert 1.6 / ent - 1 < facts["tq1_bits_per_weight"]["within_entropy_limit_percent"] / 100
    assert round(100 * (2 / ent - 1)) == facts["tq2_extra_bits_percent"]["value"]
    assert round(100 * (1 - 1.6 / 2)) == facts["tq1_saving_vs_tq2_percent"]["value"]
    assert 16 / 2 == facts["memory_bound_ceiling"]["value"]


def test_tq1_layout_and_padding():
    """Row stride, tail padding with zero trits, zero pad bytes, strict unpack."""
    assert [tq1_ldq_ref(K) for K in (5, 1024, 3072, 8192, 28672)] == [16, 208, 624, 1648, 5744]
    rng = seed_for(7, 1)
    T = ternary_iid(rng, 3, 1024, 0.3)
    qs = pack_tq1_ref(T)
    assert qs.shape == (3, 208)
    assert np.all(qs[:, 205:] == 0)
    # last group holds weights 1020..1023 and one padding trit (d' = 1, least significant)
    last = tq1_decode_division_ref(int(qs[0, 204]))
    assert last[4] == 1 and [d - 1 for d in last[:4]] == T[0, 1020:1024].tolist()
    assert np.array_equal(unpack_tq1_ref(qs, 1024), T)
    bad = qs.copy()
    bad[1, 3] = 20  # unused code
    with pytest.raises(ValueError):
        unpack_tq1_ref(bad, 1024)
    bad = qs.copy()
    bad[2, 204] = tq1_encode_group_ref((1, 1, 1, 1, 2))  # padding trit set to +1
    with pytest.raises(ValueError):
        unpack_tq1_ref(bad, 1024)


# ---------------------------------------------------------------- TQ2 codec

def test_tq2_bytes_by_hand():
    """d' = (b >> 2j) & 3 with weight 4i + j in byte i (hand-worked bytes)."""
    cases = {(1, -1, 0, 0): 0x52, (-1, 0, 1, 0): 0x64, (0, 0, 0, 0): 0x55,
             (1, 1, 1, 1): 0xAA, (-1, -1, -1, -1): 0x00}
    for w, byte in cases.items():
        qs = pack_tq2_ref(np.array([w], dtype=np.int8))
        assert int(qs[0, 0]) == byte
        assert [((byte >> (2 * j)) & 3) - 1 for j in range(4)] == list(w)
        assert unpack_tq2_ref(qs, 4).tolist() == [list(w)]
    with pytest.raises(ValueError):
        unpack_tq2_ref(np.array([[0x03]], dtype=np.uint8), 4)


def test_tq2_roundtrip_random():
    rng = seed_for(7, 2)
    T = ternary_iid(rng, 5, 512, 0.5)
    qs = pack_tq2_ref(T)
    assert qs.shape == (5, 128)
    assert np.array_equal(unpack_tq2_ref(qs, 512), T)
    # every byte of a packed ternary matrix is one of the 81 valid ones
    valid = {sum(((d + 1) << (2 * j)) for j, d in enumerate(w))
             for w in np.ndindex(3, 3, 3, 3) for w in [tuple(x - 1 for x in w)]}
    assert len(valid) == 81 and set(np.unique(qs).tolist()) <= valid


# ---------------------------------------------------------------- ternarization

def test_ternarize_hand_examples():
    T, g = ternarize_ref(np.array([[0.3, -0.05, 0.1, -0.2]]), 1e-5)
    assert abs(g - 0.16251) < 1e-12 and T.tolist() == [[1, 0, 1, -1]]
    T, g = ternarize_ref(np.array([[0.04, 0.01, -0.02, 0.005]]), 1e-5)
    assert abs(g - 0.01876) < 1e-12 and T.tolist() == [[1, 1, -1, 0]]
    # ties go to even: 1.5 is clipped to 1, 0.5 -> 0 (half away from zero would give 1)
    T, g = ternarize_ref(np.array([[3.0, 1.0]]), 0.0)
    assert g == 2.0 and T.tolist() == [[1, 0]]
    T, g = ternarize_ref(np.array([[-3.0, -1.0]]), 0.0)
    assert T.tolist() == [[-1, 0]]
    # all zero: gamma = eps, all trits zero
    T, g = ternarize_ref(np.zeros((2, 3), dtype=np.float32), 1e-5)
    assert g == 1e-5 and not T.any()
    with pytest.raises(ValueError):
        ternarize_ref(np.zeros((2, 3)), 0.0)
    with pytest.raises(ValueError):
        ternarize_ref(np.array([[1.0, np.nan]]), 1e-5)


def test_ternarize_scale_is_whole_matrix():
    """One scale per matrix: a per-row mean would ternarize row 2 to (1, -1)."""
    T, g = ternarize_ref(np.array([[0.3, 0.3], [0.01, -0.01]]), 0.0)
    assert abs(g - 0.155) < 1e-15
    assert T.tolist() == [[1, 1], [0, 0]]


def test_ternarize_sum_is_exactly_rounded():
    """|W| = (2^53, 1, 1, 0): the exact sum 2^53 + 2 is representable; a plain
    left-to-right fp64 sum would lose both ones."""
    W = np.array([[2.0 ** 53, 1.0, 1.0, 0.0]], dtype=np.float32)
    _, g = ternarize_ref(W, 0.0)
    assert g == (2.0 ** 53 + 2) / 4


def test_ternarize_gaussian_statistics():
    """N(0, s^2) latents: gamma/s -> sqrt(2/pi); P(0) = erf(1/(2 sqrt(pi))) = 0.31006."""
    W = latent_weights_f32(seed_for(7, 3), 1000, 1000, 0.02)
    T, g = ternarize_ref(W, 1e-5)
    n = T.size
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    assert abs(p0 - 0.31006) < 1e-5
    sd = math.sqrt(p0 * (1 - p0) / n)
    assert abs(np.mean(T == 0) - p0) < 5 * sd
    p1 = (1 - p0) / 2
    sd1 = math.sqrt(p1 * (1 - p1) / n)
    assert abs(np.mean(T == 1) - p1) < 5 * sd1
    assert abs((g - 1e-5) / 0.02 - math.sqrt(2 / math.pi)) < 2e-3


def test_fp16_rounding_is_one_step():
    """fp64 -> fp16 in one round-to-nearest-even step, and numpy agrees with it.

    1 + 2^-11 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-10: one
    rounding gives 1 + 2^-10; going through fp32 first would give 1.0.
    """
    x = 1 + 2.0 ** -11 + 2.0 ** -40
    assert fp16_bits_ref(x) == 0x3C01
    assert np.float16(np.float32(x)) == np.float16(1.0)
    assert np.array([x]).astype(np.float16).view(np.uint16)[0] == 0x3C01
    assert fp16_bits_ref(1 + 2.0 ** -11) == 0x3C00       # tie -> even
    assert fp16_bits_ref(1 + 3 * 2.0 ** -11) == 0x3C02   # tie -> even (up)
    assert fp16_bits_ref(2.0 ** -24) == 0x0001           # smallest subnormal
    assert fp16_bits_ref(2.0 ** -25) == 0x0000           # tie -> even (zero)
    assert fp16_bits_ref(65520.0) == 0x7C00              # rounds to infinity
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(1e-8, 1e-3, 2000), rng.uniform(0.001, 0.2, 2000),
                         rng.standard_normal(2000) * 100])
    ours = [fp16_bits_ref(float(v)) for v in xs]
    assert ours == xs.astype(np.float16).view(np.uint16).tolist()
    # struct and numpy are independent implementations of the same rounding
    assert struct.unpack("<H", struct.pack("<e", 0.1))[0] == np.float16(0.1).view(np.uint16)


# ---------------------------------------------------------------- the product

def test_gemm_special_cases():
    """Identity, minus identity, a permutation, zero, one entry per row, all ones."""
    K = 512
    X = activations_fp16(seed_for(7, 4), 3, K)
    one = np.ones((K, K // BLOCK), dtype=np.float16)
    I = np.eye(K, dtype=np.int8)
    assert np.array_equal(gemm_ref(X, I, one), X.astype(np.float64))
    assert np.array_equal(gemm_ref(X, -I, one), -X.astype(np.float64))
    perm = seed_for(7, 5).permutation(K)
    P = I[perm]  # row n has its one at column perm[n]
    assert np.array_equal(gemm_ref(X, P, one), X.astype(np.float64)[:, perm])
    assert not gemm_ref(X, np.zeros((8, K), np.int8), np.ones((8, 2), np.float16)).any()
    # one nonzero per row, block scale s[n][k//256]
    N = 6
    cols = np.array([0, 255, 256, 300, 511, 17])
    sign = np.array([1, -1, 1, -1, 1, -1])
    T = np.zeros((N, K), np.int8)
    T[np.arange(N), cols] = sign
    s = block_scales_fp16(seed_for(7, 6), N, K)
    expect = X.astype(np.float64)[:, cols] * (sign * s[np.arange(N), cols // BLOCK].astype(np.float64))
    assert np.array_equal(gemm_ref(X, T, s), expect)
    ones = np.ones((2, K), np.int8)
    assert np.array_equal(gemm_ref(X, ones, np.ones((2, 2), np.float16))[:, 0],
                          np.array([math.fsum(r) for r in X.astype(np.float64)]))


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (2, 5, 256), (3, 8, 512), (1, 7, 512)])
def test_gemm_bruteforce(M, N, K):
    rng = seed_for(7, 8, M, N, K)
    X = activations_fp16(rng, M, K)
    T = ternary_iid(rng, N, K, 0.31)
    s = block_scales_fp16(rng, N, K)
    Yb = gemm_bruteforce_ref(X, T, s)
    Y = gemm_ref(X, T, s)
    assert np.allclose(Y, Yb, rtol=1e-12, atol=1e-12)
    # column sampling gives the same numbers
    cols = np.array([N - 1, 0])
    assert np.array_equal(gemm_ref(X, T, s, cols=cols), Y[:, cols])


def test_dequantize_block_index():
    T = np.ones((1, 768), np.int8)
    s = np.array([[1.0, 2.0, 4.0]], np.float16)
    Wd = dequantize_ref(T, s)
    assert Wd[0, 255] == 1 and Wd[0, 256] == 2 and Wd[0, 511] == 2 and Wd[0, 512] == 4


# ---- SwiGLU of the decode step (gated MLP named in the architecture section)

def test_silu_closed_forms():
    """silu(0) = 0; silu(ln 3) = (3/4) ln 3 (sigmoid(ln 3) = 3/4); the odd
    identity silu(-x) = silu(x) - x; silu(x) -> x and -> 0 at the ends."""
    from oracle import silu_ref
    assert silu_ref(0.0) == 0.0
    assert abs(silu_ref(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    x = np.linspace(-30, 30, 121)
    assert np.allclose(silu_ref(-x), silu_ref(x) - x, rtol=0, atol=1e-13)
    assert silu_ref(800.0) == 800.0 and silu_ref(-800.0) == 0.0
    for v in (-7.5, -1.0, 0.25, 2.0, 9.0):
        assert abs(silu_ref(v) - v / (1.0 + math.exp(-v))) <= 1e-15 * max(1.0, abs(v))


def test_swiglu_composition():
    """Identity gate: g = x exactly, so the result is silu(x) * u; zero up
    matrix: exactly zero; brute force on a tiny random case."""
    from oracle import swiglu_ref, silu_ref
    rng = np.random.default_rng(17)
    K = 256
    X = rng.standard_normal((3, K)).astype(np.float16)
    I = np.eye(K, dtype=np.int8)
    one = np.ones((K, 1), np.float16)
    Tu = rng.integers(-1, 2, (K, K)).astype(np.int8)
    su = rng.uniform(0.5, 2, (K, 1)).astype(np.float16)
    y = swiglu_ref(X, I, one, Tu, su)
    u = gemm_ref(X, Tu, su)
    assert np.array_equal(y, silu_ref(X.astype(np.float64)) * u)
    assert not swiglu_ref(X, I, one, np.zeros((K, K), np.int8), one).any()
    N = 4
    Tg = rng.integers(-1, 2, (N, K)).astype(np.int8)
    sg = rng.uniform(0.01, 0.1, (N, 1)).astype(np.float16)
    y = swiglu_ref(X, Tg, sg, Tu[:N], su[:N])
    for m in range(3):
        for n in range(N):
            g = math.fsum(float(X[m, k]) * float(sg[n, 0]) * int(Tg[n, k]) for k in range(K))
            uu = math.fsum(float(X[m, k]) * float(su[n, 0]) * int(Tu[n, k]) for k in range(K))
            assert abs(y[m, n] - g / (1 + math.exp(-g)) * uu) <= 1e-12 * max(1.0, abs(y[m, n]))


# ---- input gradient of the ternary product (QAT backward)

def test_bwd_x_adjoint():
    """<X (sT)^T, dY> = <X, dY (sT)> for any X, dY: the backward product is
    the adjoint of gemm_ref (a transposed operand or a wrong scale index
    breaks it); identity weights give dX = dY; fsum brute force on a tiny
    case."""
    from oracle import gemm_bwd_x_ref
    rng = np.random.default_rng(23)
    M, N, K = 5, 7, 512
    T = rng.integers(-1, 2, (N, K)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, (N, K // 256)).astype(np.float16)
    X = rng.standard_normal((M, K))
    dY = rng.standard_normal((M, N))
    lhs = float(np.sum(gemm_ref(X, T, s) * dY))
    rhs = float(np.sum(X * gemm_bwd_x_ref(dY, T, s)))
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))
    I = np.eye(256, dtype=np.int8)
    d = rng.standard_normal((3, 256)).astype(np.float16)
    assert np.array_equal(gemm_bwd_x_ref(d, I, np.ones((256, 1), np.float16)), d.astype(np.float64))
    G = gemm_bwd_x_ref(dY, T, s)
    for m in range(M):
        for k in (0, 255, 256, 511):
            want = math.fsum(float(dY[m, n]) * float(s[n, k // 256]) * int(T[n, k]) for n in range(N))
            assert abs(G[m, k] - want) <= 1e-12 * max(1.0, abs(want))


def test_bwd_x_column_sampling():
    """The sampled form of the backward oracle is the full product's columns
    (block boundaries at 255/256 and the last column included)."""
    from oracle import gemm_bwd_x_ref
    rng = np.random.default_rng(81)
    N, K, M = 24, 768, 5
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    s = rng.uniform(0.01, 0.03, size=(N, K // 256)).astype(np.float16)
    dY = rng.standard_normal((M, N)).astype(np.float16)
    cols = np.array([0, 255, 256, 511, 700, K - 1])
    full = gemm_bwd_x_ref(dY, T, s)
    np.testing.assert_array_equal(gemm_bwd_x_ref(dY, T, s, cols=cols), full[:, cols])


# ---- gradient to the latent weights (straight-through estimator)

def test_ste_grad_w_adjoint_and_brute_force():
    """<X (s.T)^T, dY> = <s.T, dW> for any (T, s): the weight gradient is the
    adjoint of gemm_ref in its weight argument (a transposed operand or a
    dropped row fails it); math.fsum brute force on a tiny case; accumulation
    adds exactly."""
    from oracle import ste_grad_w_ref
    rng = np.random.default_rng(24)
    M, N, K = 6, 9, 512
    T = rng.integers(-1, 2, (N, K)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, (N, K // 256)).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    dY = rng.standard_normal((M, N)).astype(np.float16)
    G = ste_grad_w_ref(dY, X)
    assert G.shape == (N, K)
    lhs = math.fsum((gemm_ref(X, T, s) * dY.astype(np.float64)).ravel())
    rhs = math.fsum((dequantize_ref(T, s) * G).ravel())
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))
    for n in (0, 4, N - 1):
        for k in (0, 255, 256, K - 1):
            want = math.fsum(float(dY[m, n]) * float(X[m, k]) for m in range(M))
            assert abs(G[n, k] - want) <= 1e-12 * max(1.0, abs(want))
    base = rng.standard_normal((N, K)).astype(np.float32)
    np.testing.assert_array_equal(ste_grad_w_ref(dY, X, base), base.astype(np.float64) + G)
    rows = np.array([0, 3, N - 1])
    np.testing.assert_array_equal(ste_grad_w_ref(dY, X, base, rows=rows), (base + G)[rows])


def test_ste_grad_w_special_cases():
    """One activation row: dW is the outer product dY[0]^T X[0], exactly (a
    product of two fp16 values is exact in fp64).  X the identity (M = K):
    dW = dY^T.  Zero upstream gradient: dW = 0."""
    from oracle import ste_grad_w_ref
    rng = np.random.default_rng(25)
    dY = rng.standard_normal((1, 40)).astype(np.float16)
    X = rng.standard_normal((1, 256)).astype(np.float16)
    np.testing.assert_array_equal(ste_grad_w_ref(dY, X),
                                  np.outer(dY[0].astype(np.float64), X[0].astype(np.float64)))
    d = rng.standard_normal((256, 24)).astype(np.float16)
    np.testing.assert_array_equal(ste_grad_w_ref(d, np.eye(256, dtype=np.float16)),
                                  d.T.astype(np.float64))
    assert not ste_grad_w_ref(np.zeros((5, 8), np.float16), X.repeat(5, 0)).any()


def test_ste_grad_w_matches_autograd_of_the_model():
    """The layer of "The model" written in torch (fp64, CPU) with the common
    straight-through idiom W + (gamma T - W).detach(): autograd's gradient
    of <Y, dY> with respect to the latent W is ste_grad_w_ref, whatever the
    latents (so gamma is not differentiated and nothing is masked, also for
    |W / gamma| > 1)."""
    torch = pytest.importorskip("torch")
    from oracle import ste_grad_w_ref
    rng = np.random.default_rng(26)
    M, N, K = 7, 12, 256
    W0 = latent_weights_f32(rng, N, K, 0.02)
    W0[0, :8] = 0.5  # far outside the clip window
    X = rng.standard_normal((M, K)).astype(np.float16)
    dY = rng.standard_normal((M, N)).astype(np.float16)
    W = torch.tensor(W0.astype(np.float64), requires_grad=True)
    T, g = ternarize_ref(W0, 1e-5)
    q = torch.tensor(g * T.astype(np.float64))
    w_eff = W + (q - W).detach()
    Y = torch.tensor(X.astype(np.float64)) @ w_eff.T
    (Y * torch.tensor(dY.astype(np.float64))).sum().backward()
    np.testing.assert_allclose(W.grad.numpy(), ste_grad_w_ref(dY, X), rtol=0, atol=1e-12)
