"""Host ternarizer and packers of libtq.so against the oracle, bit for bit (CPU only)."""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import (
    fp16_bits_ref,
    pack_tq1_ref,
    pack_tq2_ref,
    ternarize_ref,
    tq1_decode_division_ref,
    tq1_ldq_ref,
    unpack_tq1_ref,
    unpack_tq2_ref,
)
from synth import latent_weights_f32, seed_for, ternary_iid

tq = pytest.importorskip("bit_mixed_precision_amd.binding")


def _same_gamma(a, b):
    return np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64)


# ---------------------------------------------------------------- ternarization

@pytest.mark.parametrize("N,K", [(1, 1), (3, 7), (64, 256), (257, 1024), (512, 3072)])
def test_ternarize_matches_oracle(N, K):
    W = latent_weights_f32(seed_for(11, N, K), N, K)
    T, g = tq.tq_ternarize_f32(W, 1e-5)
    Tr, gr = ternarize_ref(W, 1e-5)
    assert _same_gamma(g, gr)
    assert np.array_equal(T, Tr)


def test_ternarize_boundary_quotients():
    """W = (1, x) with eps = 0: x / gamma = 2x / (1 + x) crosses 1/2 at x = 1/3.
    Every fp32 x within 40 ulps of 1/3 must be decided the same way as the oracle."""
    x0 = np.float32(1.0 / 3.0)
    xs = [x0]
    up = dn = x0
    for _ in range(40):
        up = np.nextafter(up, np.float32(1))
        dn = np.nextafter(dn, np.float32(0))
        xs += [up, dn]
    decided = set()
    for x in xs:
        for sgn in (1, -1):
            W = np.array([[1.0, sgn * x]], dtype=np.float32)
            T, g = tq.tq_ternarize_f32(W, 0.0)
            Tr, gr = ternarize_ref(W, 0.0)
            assert _same_gamma(g, gr) and np.array_equal(T, Tr), x
            decided.add(int(T[0, 1]))
    assert decided == {-1, 0, 1}  # both sides of the boundary were exercised


def test_ternarize_ties_and_special_values():
    T, g = tq.tq_ternarize_f32(np.array([[3.0, 1.0, -3.0, -1.0]], np.float32), 0.0)
    assert g == 2.0 and T.tolist() == [[1, 0, -1, 0]]
    T, g = tq.tq_ternarize_f32(np.array([[2.0 ** 53, 1.0, 1.0, 0.0]], np.float32), 0.0)
    assert g == (2.0 ** 53 + 2) / 4
    tiny = np.array([[1e-45, 3e-39, -2e-40, 0.0, -0.0, 1e38, -3e38, 5.0]], np.float32)
    T, g = tq.tq_ternarize_f32(tiny, 1e-5)
    Tr, gr = ternarize_ref(tiny, 1e-5)
    assert _same_gamma(g, gr) and np.array_equal(T, Tr)
    for bad in (np.nan, np.inf, -np.inf):
        with pytest.raises(tq.TQError) as e:
            tq.tq_ternarize_f32(np.array([[1.0, bad]], np.float32), 1e-5)
        assert e.value.status == tq.TQ_ERR_VALUE
    with pytest.raises(tq.TQError) as e:
        tq.tq_ternarize_f32(np.zeros((2, 2), np.float32), 0.0)
    assert e.value.status == tq.TQ_ERR_VALUE


@settings(max_examples=60, deadline=None)
@given(N=st.integers(1, 9), K=st.integers(1, 40), seed=st.integers(0, 2 ** 31),
       scale=st.sampled_from([1e-30, 1e-3, 0.02, 1.0, 1e20]),
       eps=st.sampled_from([0.0, 1e-5, 0.5]))
def test_ternarize_property(N, K, seed, scale, eps):
    W = (np.random.default_rng(seed).standard_normal((N, K)) * scale).astype(np.float32)
    try:
        Tr, gr = ternarize_ref(W, eps)
    except ValueError:
        with pytest.raises(tq.TQError):
            tq.tq_ternarize_f32(W, eps)
        return
    T, g = tq.tq_ternarize_f32(W, eps)
    assert _same_gamma(g, gr) and np.array_equal(T, Tr)


def test_fp16_of_gamma_is_one_rounding():
    """W = 0 gives gamma = eps exactly, so the packed scale is fp16(eps)."""
    rng = np.random.default_rng(5)
    eps_values = [1 + 2.0 ** -11 + 2.0 ** -40, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 6.1e-5, 65504.0, 65519.99,
                  65520.0, 1e300, 1e-300, 0.1, 1 / 3]
    eps_values += list(rng.uniform(1e-9, 1e-3, 300)) + list(rng.uniform(0.005, 0.05, 300))
    eps_values += list(10.0 ** rng.uniform(-9, 4.9, 300))
    W = np.zeros((1, 256), np.float32)
    for e in eps_values:
        qs, s, g = tq.tq_pack_tq2(W, eps=e)
        assert g == e
        assert int(s.view(np.uint16)[0, 0]) == fp16_bits_ref(e), e


# ---------------------------------------------------------------- TQ2

@pytest.mark.parametrize("N,K", [(1, 256), (5, 512), (64, 1024), (300, 3072)])
def test_pack_tq2_latent(N, K):
    W = latent_weights_f32(seed_for(12, N, K), N, K)
    qs, s, g = tq.tq_pack_tq2(W, eps=1e-5)
    Tr, gr = ternarize_ref(W, 1e-5)
    assert _same_gamma(g, gr)
    assert np.array_equal(qs, pack_tq2_ref(Tr))
    assert s.shape == (N, K // 256)
    assert np.all(s.view(np.uint16) == fp16_bits_ref(gr))


@pytest.mark.parametrize("p", [0.0, 0.31, 0.9, 1.0])
def test_pack_tq2_ternary(p):
    T = ternary_iid(seed_for(13, int(p * 100)), 33, 768, p)
    qs, s, g = tq.tq_pack_tq2(T)
    assert s is None and g is None
    assert np.array_equal(qs, pack_tq2_ref(T))
    assert np.array_equal(tq.tq_unpack_tq2(qs, 768), T)
    assert np.array_equal(unpack_tq2_ref(qs, 768), tq.tq_unpack_tq2(qs, 768))


def test_pack_tq2_errors():
    T = np.zeros((2, 256), np.int8)
    T[1, 7] = 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack_tq2(T)
    assert e.value.status == tq.TQ_ERR_VALUE
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack_tq2(np.zeros((2, 100), np.int8))
    assert e.value.status == tq.TQ_ERR_SHAPE
    bad = np.full((1, 4), 0x55, np.uint8)
    bad[0, 2] = 0x57  # field 0 of byte 2 is 3
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack_tq2(bad, 16)
    assert e.value.status == tq.TQ_ERR_VALUE


# ---------------------------------------------------------------- TQ1

@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (64, 1024), (100, 3072)])
def test_pack_tq1_latent(N, K):
    W = latent_weights_f32(seed_for(14, N, K), N, K)
    qs, s, g = tq.tq_pack_tq1(W, eps=1e-5)
    Tr, gr = ternarize_ref(W, 1e-5)
    assert _same_gamma(g, gr)
    assert qs.shape == (N, tq1_ldq_ref(K)) == (N, tq.tq_tq1_ldq(K))
    assert np.array_equal(qs, pack_tq1_ref(Tr))
    assert np.all(s.view(np.uint16) == fp16_bits_ref(gr))


@pytest.mark.parametrize("p", [0.3, 0.5, 0.9])
@pytest.mark.parametrize("ldq_extra", [0, 16, 48])
def test_pack_tq1_ternary(p, ldq_extra):
    K = 1024
    T = ternary_iid(seed_for(15, int(p * 10), ldq_extra), 21, K, p)
    ldq = tq1_ldq_ref(K) + ldq_extra
    qs, _, _ = tq.tq_pack_tq1(T, ldq=ldq)
    assert np.array_equal(qs, pack_tq1_ref(T, ldq))
    assert np.array_equal(tq.tq_unpack_tq1(qs, K), T)
    assert np.array_equal(unpack_tq1_ref(qs, K, ldq), T)


def test_pack_tq1_minimal_ldq():
    K = 256  # ceil(256/5) = 52 bytes, not a multiple of 16: allowed for packing
    T = ternary_iid(seed_for(16), 4, K, 0.3)
    qs, _, _ = tq.tq_pack_tq1(T, ldq=52)
    assert np.array_equal(qs, pack_tq1_ref(T, 52))
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack_tq1(T, ldq=51)
    assert e.value.status == tq.TQ_ERR_SHAPE


def test_unpack_tq1_every_byte():
    """One group per row (K = 5): valid bytes decode as the division route does,
    the 13 unused ones are rejected."""
    for b in range(256):
        qs = np.zeros((1, 16), np.uint8)
        qs[0, 0] = b
        ref = tq1_decode_division_ref(b)
        if ref is None:
            with pytest.raises(tq.TQError) as e:
                tq.tq_unpack_tq1(qs, 5)
            assert e.value.status == tq.TQ_ERR_VALUE
        else:
            assert tq.tq_unpack_tq1(qs, 5)[0].tolist() == [d - 1 for d in ref]


def test_unpack_tq1_padding_trit():
    T = ternary_iid(seed_for(17), 2, 1024, 0.3)
    qs, _, _ = tq.tq_pack_tq1(T)
    g = 1024 // 5  # the last group holds weights 1020..1023 and one padding trit
    qs[1, g] = qs[1, g] + 1 if tq1_decode_division_ref(int(qs[1, g]) + 1) else qs[1, g] - 1
    with pytest.raises(tq.TQError):
        tq.tq_unpack_tq1(qs, 1024)


@pytest.mark.slow
def test_pack_full_size_latent():
    """The largest latent shape of the workloads (8192 x 8192 here): gamma and bytes."""
    N = K = 8192
    W = latent_weights_f32(seed_for(18), N, K)
    qs2, s2, g = tq.tq_pack_tq2(W, eps=1e-5)
    Tr, gr = ternarize_ref(W, 1e-5)
    assert _same_gamma(g, gr)
    assert np.array_equal(qs2, pack_tq2_ref(Tr))
    qs1, _, _ = tq.tq_pack_tq1(Tr)
    assert np.array_equal(qs1, pack_tq1_ref(Tr))
    assert abs(np.mean(Tr == 0) - math.erf(1 / (2 * math.sqrt(math.pi)))) < 1e-3
