"""On-device ternarize + pack (tq_pack_tq2_dev / tq_pack_tq1_dev) against the
host packer and the oracle: gamma, qs and scales must be identical bit for bit.

Cases: N(0, 0.02) latents at several shapes (ragged N, K from one to many
blocks, TQ1 with a wider ldq), exact ties W / gamma = +-1/2 (round to even
leaves 0), an all-zero matrix (gamma = eps), fp32 subnormals next to large
values (the exact sum must not lose them), and a non-finite latent (status).
"""

import sys

import numpy as np
import pytest

from oracle import pack_tq1_ref, pack_tq2_ref, ternarize_ref
from synth import latent_weights_f32, seed_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("bit_mixed_precision_amd.binding")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def device_pack(fmt, W, eps, ldq=None):
    Wd = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    qs, sc, g, st = tq.tq_pack_dev(fmt, Wd, eps, ldq)
    torch.cuda.synchronize()
    return qs.cpu().numpy(), sc.cpu().numpy().view(np.uint16), float(g.item()), int(st.item())


def host_pack(fmt, W, eps, ldq=None):
    if fmt == 2:
        qs, sc, g = tq.tq_pack_tq2(W, eps)
    else:
        qs, sc, g = tq.tq_pack_tq1(W, eps, ldq)
    return qs, sc.view(np.uint16), g


@pytest.mark.parametrize("fmt", [2, 1])
@pytest.mark.parametrize("N,K,ldq", [(1, 256, None), (37, 512, None), (100, 1024, 240),
                                     (100, 1024, 237), (777, 2560, None), (4096, 8192, None)])
def test_device_pack_matches_host(fmt, N, K, ldq):
    say(f"[pack] fmt={fmt} N={N} K={K} ldq={ldq}")
    W = latent_weights_f32(seed_for(80, N, K), N, K)
    ldq = ldq if fmt == 1 else None
    qs, sc, g, st = device_pack(fmt, W, 1e-5, ldq)
    hq, hs, hg = host_pack(fmt, W, 1e-5, ldq)
    assert st == tq.TQ_OK
    assert g == hg  # exact
    assert np.array_equal(qs, hq)
    assert np.array_equal(sc, hs)


@pytest.mark.parametrize("fmt", [2, 1])
def test_device_pack_matches_oracle_small(fmt):
    N, K = 8, 512
    W = latent_weights_f32(seed_for(81, N, K), N, K)
    qs, sc, g, st = device_pack(fmt, W, 1e-5)
    T, gamma = ternarize_ref(W, 1e-5)
    assert st == tq.TQ_OK and g == gamma
    ref = pack_tq2_ref(T) if fmt == 2 else pack_tq1_ref(T)
    assert np.array_equal(qs, ref)


@pytest.mark.parametrize("fmt", [2, 1])
def test_device_pack_ties_zero_and_extremes(fmt):
    K = 256
    # mean |W| = 2 with eps = 0: W / gamma hits 1.5, 0.5, -0.5, -1.5 exactly
    pattern = np.array([3, 1, -1, -3], dtype=np.float32)
    W = np.tile(pattern, (3, K // 4))
    qs, sc, g, st = device_pack(fmt, W, 0.0)
    hq, hs, hg = host_pack(fmt, W, 0.0)
    assert st == tq.TQ_OK and g == 2.0 == hg
    assert np.array_equal(qs, hq) and np.array_equal(sc, hs)
    if fmt == 2:
        assert qs[0, 0] == (2 | (1 << 2) | (1 << 4) | (0 << 6))  # trits 1, 0, 0, -1
    # all zero: gamma = eps, every trit 0
    Z = np.zeros((2, K), dtype=np.float32)
    qs, sc, g, st = device_pack(fmt, Z, 1e-3)
    assert st == tq.TQ_OK and g == 1e-3
    assert np.array_equal(qs, host_pack(fmt, Z, 1e-3)[0])
    # subnormals and large values: the exact sum keeps every bit
    E = latent_weights_f32(seed_for(82, 4, K), 4, K)
    E[0, :16] = np.float32(1e-42)
    E[1, :8] = np.float32(3e30)
    E[2, :4] = -np.float32(1.1754942e-38)
    qs, sc, g, st = device_pack(fmt, E, 1e-5)
    hq, hs, hg = host_pack(fmt, E, 1e-5)
    assert st == tq.TQ_OK and g == hg
    assert np.array_equal(qs, hq) and np.array_equal(sc, hs)


@pytest.mark.parametrize("fmt", [2, 1])
def test_device_pack_non_finite_status(fmt):
    W = latent_weights_f32(seed_for(83, 4, 256), 4, 256)
    W[2, 7] = np.inf
    _, _, _, st = device_pack(fmt, W, 1e-5)
    assert st == tq.TQ_ERR_VALUE
    W[2, 7] = np.nan
    _, _, _, st = device_pack(fmt, W, 1e-5)
    assert st == tq.TQ_ERR_VALUE
