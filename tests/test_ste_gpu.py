"""GPU parity of the latent-weight gradient (straight-through estimator):
tq_ste_grad_w through the C ABI against the fp64 oracle ste_grad_w_ref.

Bar: max|dW - dW_ref| <= 4e-3 * max|dW_ref| (the product's tolerance; the
output here is fp32, so the error is logged in units of max|dW_ref| too);
exact where every partial sum is exact in fp32 (small integers).
"""

import sys

import numpy as np
import pytest

from gpu_util import activations, strat_cols
from oracle import ste_grad_w_ref

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("bit_mixed_precision_amd.binding")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_f32(G, R, label):
    G64, R64 = np.asarray(G, np.float64), np.asarray(R, np.float64)
    assert G64.shape == R64.shape and np.all(np.isfinite(G64)), label
    big = float(np.max(np.abs(R64))) if R64.size else 0.0
    err = float(np.max(np.abs(G64 - R64))) if R64.size else 0.0
    assert err <= 4e-3 * big or (big == 0.0 and err == 0.0), (label, err, big)
    say(f"  {label}: max err / max|ref| = {err / big if big else 0.0:.2e}")


# ragged in every dimension: M against the 32-row step, N and K against the
# 256 x 256 tile and its 32-wide MFMA blocks
SHAPES = [(1, 8, 8), (5, 40, 264), (33, 264, 520), (64, 256, 256), (100, 512, 1032),
          (257, 1000, 1288), (31, 2056, 72)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_ste_grad_w_parity(M, N, K):
    say(f"[ste] M={M} N={N} K={K}")
    dY, X = activations(M, N, 121), activations(M, K, 122)
    dW = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_ste_grad_w(dev(dY), dev(X), dW)
    torch.cuda.synchronize()
    check_f32(dW.cpu().numpy(), ste_grad_w_ref(dY, X), f"ste {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(5, 40, 264), (257, 1000, 1288)])
def test_ste_grad_w_accumulate(M, N, K):
    """accumulate = 1 adds to the gradient already there (micro-batches):
    two halves of a batch accumulated equal the oracle on the whole batch."""
    say(f"[ste acc] M={M} N={N} K={K}")
    dY, X = activations(M, N, 123), activations(M, K, 124)
    base = np.random.default_rng(125).standard_normal((N, K)).astype(np.float32)
    dW = dev(base)
    h = M // 2
    tq.tq_ste_grad_w(dev(dY[:h]), dev(X[:h]), dW, accumulate=True)
    tq.tq_ste_grad_w(dev(dY[h:]), dev(X[h:]), dW, accumulate=True)
    torch.cuda.synchronize()
    check_f32(dW.cpu().numpy(), ste_grad_w_ref(dY, X, base), f"ste acc {M}x{N}x{K}")


def test_ste_grad_w_exact_integers_and_empty_batch():
    """Integer dY and X in [-3, 3]: every partial sum is an integer below 2^24,
    so dW equals the oracle exactly.  M = 0 writes zeros; with accumulate it
    leaves dW as it was."""
    M, N, K = 300, 264, 520
    rng = np.random.default_rng(126)
    dY = rng.integers(-3, 4, size=(M, N)).astype(np.float16)
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    G = tq.tq_ste_grad_w(dev(dY), dev(X)).cpu().numpy()
    np.testing.assert_array_equal(G.astype(np.float64), ste_grad_w_ref(dY, X))
    z = dev(np.zeros((0, N), np.float16)), dev(np.zeros((0, K), np.float16))
    dW = torch.full((N, K), 5.0, dtype=torch.float32, device="cuda")
    tq.tq_ste_grad_w(*z, dW, accumulate=True)
    torch.cuda.synchronize()
    assert bool((dW == 5.0).all())
    tq.tq_ste_grad_w(*z, dW)
    torch.cuda.synchronize()
    assert bool((dW == 0.0).all())


def test_ste_grad_w_deterministic():
    M, N, K = 1000, 768, 1024
    dY, X = dev(activations(M, N, 127)), dev(activations(M, K, 128))
    a = tq.tq_ste_grad_w(dY, X)
    b = tq.tq_ste_grad_w(dY, X)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_ste_grad_w_full_size():
    """The bench's launch: 4096 tokens, N = K = 8192; every column k of rows n
    stratified over the whole height (one in every 16, both edges of every
    32-row block) against the oracle."""
    M, N, K = 4096, 8192, 8192
    say(f"[ste full] M={M} N={N} K={K}")
    dY, X = activations(M, N, 129), activations(M, K, 130)
    dW = tq.tq_ste_grad_w(dev(dY), dev(X))
    torch.cuda.synchronize()
    rows = strat_cols(N, 131)
    sel = torch.from_numpy(rows).cuda()
    check_f32(dW[sel].cpu().numpy(), ste_grad_w_ref(dY, X, rows=rows), "ste full")
