"""GPU parity of the table-decode TQ1 tiled kernel (tq_gemm_tq1_tile and the
automatic TQ1 choice that uses it) against the fp64 oracle.

The kernel copies each 256-weight block's TQ1 bytes to LDS and rebuilds the
block's 2-bit fields from a byte table, so the cases cover every trit offset a
block can start at (block b starts at trit b mod 5 of its first byte: K with
five or more blocks), blocks fewer than the k-groups, ragged M and N, and a
row stride larger than ceil(K / 5).  Bar: max|Y - Y_ref| <= 4e-3 max|Y_ref|,
and bit-exact fp16 where the exact product is representable.
"""

import sys

import numpy as np
import pytest

from gpu_util import DenseRef, activations, check_close, iid_problem, ref

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("bit_mixed_precision_amd.binding")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_out(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")


TILES = [(mt, 4, ng, kg) for mt in (2, 4) for ng, kg in ((4, 2), (2, 4), (2, 2), (1, 4))]
TILES += [(mt, 2, ng, 4) for mt in (2, 4) for ng in (1, 2)]
TILES.append((8, 2, 4, 2))
TILES += [(2, 2, 1, 8), (2, 4, 1, 8)]
# (M, N, K, ldq): K / 256 = 1, 3, 5, 7, 2, 112 (every block trit offset 0..4
# from five blocks on; fewer blocks than k-groups; the down projection's
# K = 28672, where byte offsets within a row pass 2^12); ldq above ceil(K / 5)
TAB_SHAPES = [(17, 100, 256, None), (40, 300, 768, None), (64, 257, 1280, 272),
              (100, 520, 1792, None), (130, 70, 512, 128), (33, 72, 28672, 5760)]


@pytest.mark.parametrize("mt,nr,ng,kg", TILES)
@pytest.mark.parametrize("M,N,K,ldq", TAB_SHAPES)
def test_every_tq1_tab_tile(mt, nr, ng, kg, M, N, K, ldq):
    say(f"[tq1 tab] mt={mt} nr={nr} ng={ng} kg={kg} M={M} N={N} K={K} ldq={ldq}")
    T, s = iid_problem(N, K, 0.31, 21)
    X = activations(M, K, 21)
    ldq = ldq or tq.tq_tq1_ldq(K)
    q = tq.tq_pack_tq1(T, ldq=ldq)[0]
    Y = nan_out(M, N)
    tq.tq_gemm_tq1_tile(dev(X), dev(q), dev(s), mt, nr, ng, kg, Y)
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), ref(X, T, s), f"tq1 tab {mt},{nr},{ng},{kg} {M}x{N}x{K}")


@pytest.mark.parametrize("tile", [(2, 2, 1, 8), (4, 4, 2, 4), (8, 2, 4, 2)])
def test_tq1_tab_exact_special_cases(tile):
    """Identity, minus identity and a permutation with unit scales: every
    output is one activation, so the fp16 bits must equal it (both the
    block-sum and the scale-in-operand variants are exact here)."""
    K = 1280  # five blocks: every trit offset of a block start
    X = activations(40, K, 22)
    one = np.ones((K, K // 256), np.float16)
    I = np.eye(K, dtype=np.int8)
    perm = np.random.default_rng(23).permutation(K)
    for W, want in ((I, X), (-I, -X), (I[perm], X[:, perm])):
        q = tq.tq_pack_tq1(W)[0]
        Y = tq.tq_gemm_tq1_tile(dev(X), dev(q), dev(one), *tile).cpu().numpy()
        assert np.array_equal(Y.astype(np.float64), want.astype(np.float64)), tile


def test_tq1_tab_refuses_uncompiled_tile_and_huge_ldq():
    M, N, K = 32, 64, 256
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    q = torch.zeros((N, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((N, 1), dtype=torch.float16, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    st = tq.lib.tq_gemm_tq1_tile(X.data_ptr(), q.data_ptr(), 64, s.data_ptr(), Y.data_ptr(), M, N,
                                 K, 3, 4, 2, 4, None)
    assert st == tq.TQ_ERR_UNSUPPORTED
    st = tq.lib.tq_gemm_tq1_tile(X.data_ptr(), q.data_ptr(), (1 << 22) + 16, s.data_ptr(),
                                 Y.data_ptr(), M, N, K, 2, 4, 1, 8, None)
    assert st == tq.TQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())


@pytest.mark.parametrize("N", [8192, 28672])
def test_tq1_tab_full_size_every_column(N):
    """K = 8192 at M = 32, 64, 128 on the tile the automatic TQ2 choice takes
    for that shape, every output column against the oracle."""
    K = 8192
    T, s = iid_problem(N, K, 0.5, 24)
    q = tq.tq_pack_tq1(T)[0]
    qd, sd = dev(q), dev(s)
    R = DenseRef(T, s)
    del T
    for M in (32, 64, 128):
        X = activations(M, K, 24 + M)
        Y = nan_out(M, N)
        name = tq.tq_kernel_name(2, M, N, K, 2)  # the TQ2 tiled choice for this shape
        tile = tuple(int(v) for v in name[name.index("<") + 1:-1].split(","))
        say(f"[tq1 tab full] N={N} M={M} tile={tile}")
        tq.tq_gemm_tq1_tile(dev(X), qd, sd, *tile, Y)
        torch.cuda.synchronize()
        check_close(Y.cpu().numpy(), R(X), f"tq1 tab full N={N} M={M}")


def test_tq1_auto_large_row_stride_runs_skinny():
    """ldq past 2^22 (a 4 MiB row stride): the automatic choice at M > 16
    takes the skinny kernel, whose offsets allow it, and stays exact to the
    bar; the explicit table-kernel entry refuses it."""
    M, N, K = 40, 16, 512
    ldq = (1 << 22) + 16
    T, s = iid_problem(N, K, 0.31, 25)
    X = activations(M, K, 25)
    q = tq.tq_pack_tq1(T, ldq=ldq)[0]
    Y = tq.tq_gemm_tq1(dev(X), dev(q), dev(s))
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), ref(X, T, s), "tq1 auto, ldq = 2^22 + 16")
