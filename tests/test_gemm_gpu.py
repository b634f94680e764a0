"""GPU parity: tq_gemm_tq2 / tq_gemm_tq1 through the C ABI against the fp64 oracle.

Bar: max|Y - Y_ref| <= 4e-3 * max|Y_ref| (Y is the fp16 GPU output widened to
fp64); exact equality where the product is exactly representable (identity,
permutations, one weight per row, zero weights), except for the stated fp32
rounding of the folded d' = d + 1 offset on the skinny paths.  Every kernel family is forced
at every M through the *_ex entry points, so both sides of the M switch are
covered.
"""

import sys

import numpy as np
import pytest

from gpu_util import DenseRef, activations, check_close, iid_problem, ref, strat_cols
from oracle import pack_tq1_ref, pack_tq2_ref, ternarize_ref
from synth import latent_weights_f32, seed_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("bit_mixed_precision_amd.binding")

PATHS = {"simple": 3, "skinny": 1, "tiled": 2, "auto": 0}
SKINNY_MAX_M = 32


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def run(fmt, X, qs, s, path, Y=None):
    Xd, qd, sd = (x if torch.is_tensor(x) else dev(x) for x in (X, qs, s))
    if Y is None:  # NaN sentinel: an output the kernel does not write fails the check
        Y = torch.full((Xd.shape[0], qd.shape[0]), float("nan"), dtype=torch.float16,
                       device=Xd.device)
    if fmt == "tq2":
        Yd = tq.tq_gemm_tq2_ex(Xd, qd, sd, PATHS[path], Y)
    else:
        Yd = tq.tq_gemm_tq1_ex(Xd, qd, sd, PATHS[path], Y)
    torch.cuda.synchronize()
    return Yd


def pack(fmt, T):
    if fmt == "tq2":
        return tq.tq_pack_tq2(T)[0]
    return tq.tq_pack_tq1(T)[0]


def supported(fmt, path):
    X = torch.zeros((1, 256), dtype=torch.float16, device="cuda")
    s = torch.ones((16, 1), dtype=torch.float16, device="cuda")
    q = torch.zeros((16, 64 if fmt == "tq2" else 64), dtype=torch.uint8, device="cuda")
    Y = torch.empty((1, 16), dtype=torch.float16, device="cuda")
    fn = tq.lib.tq_gemm_tq2_ex if fmt == "tq2" else None
    if fmt == "tq2":
        st = fn(X.data_ptr(), q.data_ptr(), s.data_ptr(), Y.data_ptr(), 1, 16, 256, PATHS[path],
                None)
    else:
        st = tq.lib.tq_gemm_tq1_ex(X.data_ptr(), q.data_ptr(), 64, s.data_ptr(), Y.data_ptr(), 1,
                                   16, 256, PATHS[path], None)
    torch.cuda.synchronize()
    return st != tq.TQ_ERR_UNSUPPORTED


def need(fmt, path):
    if not supported(fmt, path):
        pytest.skip(f"{path} kernel family not available for {fmt}")


SMALL = [(1, 1024, 1024), (2, 48, 512), (3, 100, 768), (4, 17, 256), (5, 64, 256),
         (6, 33, 512), (7, 31, 768), (8, 130, 1280), (12, 80, 768), (13, 16, 256),
         (9, 64, 512), (16, 257, 2048), (17, 96, 768), (32, 40, 1024), (33, 200, 512),
         (64, 128, 1536), (100, 77, 256), (128, 300, 1024)]


# Every (format, family) at every small shape, except the TQ2 skinny family
# past its M <= 32 limit (it refuses such calls: TQ_ERR_UNSUPPORTED, which
# test_skinny_tq2_refuses_large_m checks), so that a skip always means something.
SMALL_CASES = [(fmt, path, M, N, K) for M, N, K in SMALL for fmt in ("tq2", "tq1")
               for path in ("simple", "skinny", "tiled", "auto")
               if not (fmt == "tq2" and path == "skinny" and M > SKINNY_MAX_M)]


@pytest.mark.parametrize("fmt,path,M,N,K", SMALL_CASES)
def test_small_parity(fmt, path, M, N, K):
    need(fmt, path)
    say(f"[small] {fmt} {path} M={M} N={N} K={K}")
    T, s = iid_problem(N, K, 0.31, 1)
    X = activations(M, K, 1)
    Y = run(fmt, X, pack(fmt, T), s, path).cpu().numpy()
    check_close(Y, ref(X, T, s), f"{fmt}/{path}/{M}x{N}x{K}")


# Skinny TQ2 shapes whose activations need several LDS windows: a short last
# window in which some waves have no block (K = 5120, 9216, 6400), nb not a
# multiple of the waves per row group, and seven windows (K = 28672); with two
# m tiles (M = 17 .. 32): windows of 8 blocks, a second m tile of one row
# (M = 17), more row groups than a workgroup of two m tiles takes (N = 40000:
# 10 row groups per CU, run as 8), and block scales loaded with each pair
# instead of staged (N = 30000, K = 8448: 8 row groups x 33 blocks is more
# than four scales per thread; an odd block count leaves the last pair half
# empty).
SKINNY_WINDOWS = [(16, 300, 5120), (16, 300, 28672), (9, 8192, 9216), (13, 1000, 6400),
                  (32, 300, 5120), (17, 1000, 6400), (24, 2048, 8192), (32, 2048, 8192),
                  (20, 40000, 512), (20, 30000, 8448)]


@pytest.mark.parametrize("M,N,K", SKINNY_WINDOWS)
def test_skinny_windows(M, N, K):
    say(f"[windows] tq2 skinny M={M} N={N} K={K}")
    T, s = iid_problem(N, K, 0.31, 5)
    X = activations(M, K, 5)
    Y = run("tq2", X, pack("tq2", T), s, "skinny").cpu().numpy()
    check_close(Y, ref(X, T, s), f"windows {M}x{N}x{K}")


def test_skinny_tq2_refuses_large_m():
    """The TQ2 skinny family serves M <= 32 only: a forced call past it returns
    TQ_ERR_UNSUPPORTED and writes nothing."""
    M, N, K = 33, 64, 256
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    q = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    s = torch.ones((N, 1), dtype=torch.float16, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    st = tq.lib.tq_gemm_tq2_ex(X.data_ptr(), q.data_ptr(), s.data_ptr(), Y.data_ptr(), M, N, K,
                               PATHS["skinny"], None)
    torch.cuda.synchronize()
    assert st == tq.TQ_ERR_UNSUPPORTED
    assert bool((Y == 7.0).all())


TILES = [(mt, 4, ng, kg) for mt in (2, 4) for ng, kg in ((4, 2), (2, 4), (2, 2), (1, 4))]
TILES += [(mt, 2, ng, 4) for mt in (2, 4) for ng in (1, 2)]  # 32 weight rows per wave
TILES.append((8, 2, 4, 2))  # 128 activation rows x 32 weight rows per wave
TILES += [(2, 2, 1, 8), (2, 4, 1, 8)]  # 32 x 32 and 32 x 64 over 8 k-groups
# ragged in M and N, K / 256 = 1, 2, 3, 5 (fewer blocks than k-groups, odd counts)
TILE_SHAPES = [(17, 100, 256), (40, 300, 768), (64, 257, 1024), (100, 520, 1280),
               (130, 1000, 512)]


@pytest.mark.parametrize("mt,nr,ng,kg", TILES)
@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_every_tiled_tile(mt, nr, ng, kg, M, N, K):
    """Each compiled tile of the tiled kernel, not only the ones the shape
    heuristic picks, over several tiles and ragged tails (tiles with the
    default weight rows per wave also through tq_gemm_tq2_tiled)."""
    say(f"[tile] mt={mt} nr={nr} ng={ng} kg={kg} M={M} N={N} K={K}")
    T, s = iid_problem(N, K, 0.31, 5)
    X = activations(M, K, 5)
    Xd, qd, sd = dev(X), dev(pack("tq2", T)), dev(s)
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tq.tq_gemm_tq2_tile(Xd, qd, sd, mt, nr, ng, kg, Y)
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), ref(X, T, s), f"tile {mt},{nr},{ng},{kg} {M}x{N}x{K}")
    if nr == (2 if mt == 8 else 4):
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        tq.tq_gemm_tq2_tiled(Xd, qd, sd, mt, ng, kg, Y)
        torch.cuda.synchronize()
        check_close(Y.cpu().numpy(), ref(X, T, s), f"tiled {mt},{ng},{kg} {M}x{N}x{K}")


WIDE_TILES = [(mt, nt, 2, 2) for mt in (1, 2, 4) for nt in (1, 2)]
WIDE_TILES += [(mt, nt, 1, 4) for mt in (1, 2) for nt in (1, 2)]
# ragged in M and N against the 32-row blocks and the tiles; K / 256 = 1 .. 5
# (one stage to several), M = 1 (one real row in a 32-row block)
WIDE_SHAPES = [(1, 64, 256), (17, 100, 256), (40, 300, 768), (64, 257, 1024),
               (100, 520, 1280), (130, 1000, 512)]


@pytest.mark.parametrize("mt,nt,ng,kg", WIDE_TILES)
@pytest.mark.parametrize("M,N,K", WIDE_SHAPES)
def test_every_wide_tile(mt, nt, ng, kg, M, N, K):
    """Each compiled tile of the wide-tile (32 x 32 x 16 MFMA) kernel over
    several tiles and ragged tails against the oracle."""
    say(f"[wide] mt={mt} nt={nt} ng={ng} kg={kg} M={M} N={N} K={K}")
    T, s = iid_problem(N, K, 0.31, 15)
    X = activations(M, K, 15)
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tq.tq_gemm_tq2_wide(dev(X), dev(pack("tq2", T)), dev(s), mt, nt, ng, kg, Y)
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), ref(X, T, s), f"wide {mt},{nt},{ng},{kg} {M}x{N}x{K}")


def test_wide_exact_special_cases():
    """The wide kernel decodes exact trits times the block scale: identity,
    minus identity, a permutation and one weight per row give fp16 bits equal
    to the exact product's rounding."""
    K = 512
    for tile in ((4, 2, 2, 2), (1, 1, 1, 4)):
        X = activations(40, K, 16)
        one = np.ones((K, K // 256), np.float16)
        I = np.eye(K, dtype=np.int8)
        for W, want in ((I, X), (-I, -X)):
            Y = tq.tq_gemm_tq2_wide(dev(X), dev(pack("tq2", W)), dev(one), *tile).cpu().numpy()
            assert np.array_equal(Y.astype(np.float64), want.astype(np.float64)), tile
        perm = seed_for(17).permutation(K)
        Y = tq.tq_gemm_tq2_wide(dev(X), dev(pack("tq2", I[perm])), dev(one), *tile).cpu().numpy()
        assert np.array_equal(Y.view(np.uint16), X[:, perm].view(np.uint16)), tile


def ulp16(v):
    """Spacing of fp16 numbers at |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def same_or_offset_bound(Y, want, X, smax, fmt, path, bits=True):
    """Bit-exact, except on the skinny paths: their decoders leave the stored
    digit d' = d + 1 and subtract the block (TQ2) or span (TQ1) sums of the
    activations in fp32, so a result carries the rounding of that
    cancellation, at most 2^-16 * max|s| * sum_k |x[m, k]| per row m (the
    derivation gives about 2^-19), besides the fp16 rounding of the output."""
    Y64, want64 = Y.astype(np.float64), np.asarray(want, np.float64)
    if path != "skinny":
        if bits:  # same fp16 bit patterns (+0 where want is +0)
            assert np.array_equal(Y.view(np.uint16), np.asarray(want, np.float16).view(np.uint16))
        else:  # same values (either sign of zero)
            assert np.array_equal(Y64, want64)
        return
    bound = 2.0 ** -16 * smax * np.abs(X.astype(np.float64)).sum(axis=1, keepdims=True)
    err = np.abs(Y64 - want64)
    assert np.all(err <= 0.5 * ulp16(want64) + bound), float(np.max(err - bound))


@pytest.mark.parametrize("path", ["simple", "skinny", "tiled"])
@pytest.mark.parametrize("fmt", ["tq2", "tq1"])
def test_exact_special_cases(fmt, path):
    """Identity, minus identity, permutation, zero, one weight per row: exact
    (up to the stated offset rounding on the skinny paths)."""
    need(fmt, path)
    K = 512
    for M in (1, 5, 16, 29, 40):
        if path == "skinny" and fmt == "tq2" and M > SKINNY_MAX_M:
            continue
        say(f"[exact] {fmt} {path} M={M}")
        X = activations(M, K, 2)
        one = np.ones((K, K // 256), np.float16)
        I = np.eye(K, dtype=np.int8)
        Y = run(fmt, X, pack(fmt, I), one, path).cpu().numpy()
        same_or_offset_bound(Y, X, X, 1.0, fmt, path)
        Y = run(fmt, X, pack(fmt, -I), one, path).cpu().numpy()
        same_or_offset_bound(Y, -X, X, 1.0, fmt, path, bits=False)
        perm = seed_for(3).permutation(K)
        Y = run(fmt, X, pack(fmt, I[perm]), one, path).cpu().numpy()
        same_or_offset_bound(Y, X[:, perm], X, 1.0, fmt, path)
        Z = np.zeros((48, K), np.int8)
        Y = run(fmt, X, pack(fmt, Z), np.ones((48, 2), np.float16), path).cpu().numpy()
        same_or_offset_bound(Y, np.zeros((M, 48)), X, 1.0, fmt, path)  # +0 everywhere
        # one nonzero per row with block scales: Y = fp16(+-x * s), exact product
        N = 64
        cols = seed_for(4).integers(0, K, N)
        sign = np.where(seed_for(5).random(N) < 0.5, -1, 1).astype(np.int8)
        T = np.zeros((N, K), np.int8)
        T[np.arange(N), cols] = sign
        s = iid_problem(N, K, 0.31, 6)[1]
        Y = run(fmt, X, pack(fmt, T), s, path).cpu().numpy()
        want = ref(X, T, s).astype(np.float16)  # exact product, one rounding
        same_or_offset_bound(Y, want, X, float(np.abs(s.astype(np.float64)).max()), fmt, path)


@pytest.mark.parametrize("path", ["simple", "skinny", "tiled"])
def test_tq1_ragged_tail(path):
    """K = 256, 768, 1280: 5 does not divide K, the last group carries padding."""
    need("tq1", path)
    for K in (256, 768, 1280, 3072):
        T, s = iid_problem(40, K, 0.5, 7)
        T = T.copy()
        T[:, -1] = 1  # the last real weight of each row is non-zero
        X = activations(3, K, 7)
        Y = run("tq1", X, pack("tq1", T), s, path).cpu().numpy()
        check_close(Y, ref(X, T, s), f"tq1 tail K={K}")


def test_cross_format_same_weights():
    """TQ2 and TQ1 packings of the same (T, s) give the same Y_ref, and both GPU
    results meet the bar."""
    N, K = 512, 2048
    for p in (0.3, 0.5, 0.9):
        T, s = iid_problem(N, K, p, 8)
        for M in (1, 4, 16, 64):
            X = activations(M, K, 8)
            R = ref(X, T, s)
            Y2 = run("tq2", X, pack("tq2", T), s, "auto").cpu().numpy()
            Y1 = run("tq1", X, pack("tq1", T), s, "auto").cpu().numpy()
            check_close(Y2, R, f"tq2 p={p} M={M}")
            check_close(Y1, R, f"tq1 p={p} M={M}")


def test_deterministic_bits():
    T, s = iid_problem(1024, 4096, 0.31, 9)
    q2, q1 = dev(pack("tq2", T)), dev(pack("tq1", T))
    sd = dev(s)
    for M in (1, 8, 16, 64):
        X = dev(activations(M, 4096, 9))
        a = run("tq2", X, q2, sd, "auto").clone()
        b = run("tq2", X, q2, sd, "auto")
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        a = run("tq1", X, q1, sd, "auto").clone()
        b = run("tq1", X, q1, sd, "auto")
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_latent_end_to_end():
    """Latents -> host packer -> GPU, against the oracle's own ternarization.
    Shapes: the 1024 x 1024 layer and the 3B-class decode linears at M = 1."""
    shapes = [(1024, 1024), (3072, 3072), (3072, 8192), (8192, 3072)]
    for i, (K, N) in enumerate(shapes):
        say(f"[latent] K={K} N={N}")
        W = latent_weights_f32(seed_for(20, i), N, K, 0.02)
        Tr, g = ternarize_ref(W, 1e-5)
        X = activations(1, K, 20 + i)
        s_ref = np.full((N, K // 256), np.float16(g))
        R = ref(X, Tr, s_ref)
        q2, s2, _ = tq.tq_pack_tq2(W, eps=1e-5)
        assert np.array_equal(q2, pack_tq2_ref(Tr))
        check_close(run("tq2", X, q2, s2, "auto").cpu().numpy(), R, f"latent tq2 {K}x{N}")
        q1, s1, _ = tq.tq_pack_tq1(W, eps=1e-5)
        assert np.array_equal(q1, pack_tq1_ref(Tr))
        check_close(run("tq1", X, q1, s1, "auto").cpu().numpy(), R, f"latent tq1 {K}x{N}")


FULL_M = [1, 2, 4, 8, 16, 20, 32, 64, 128]


@pytest.mark.parametrize("N", [8192, 28672])
def test_full_size_tq2_sweep(N):
    """The K = 8192 batch sweep at full size on the automatic kernel choice
    (the launches the bench times): every output column of every M against
    the oracle, so every weight-row tile, tile order and XCD mapping of the
    skinny and tiled kernels is checked."""
    K = 8192
    T, s = iid_problem(N, K, 0.31, 30)
    qd, sd = dev(pack("tq2", T)), dev(s)
    R = DenseRef(T, s)
    for M in FULL_M:
        say(f"[full tq2] N={N} M={M} {tq.tq_kernel_name(2, M, N, K)}")
        X = activations(M, K, 30 + M)
        Y = run("tq2", X, qd, sd, "auto").cpu().numpy()
        check_close(Y, R(X), f"full tq2 N={N} M={M}")


@pytest.mark.parametrize("N", [8192, 28672])
@pytest.mark.parametrize("p", [0.3, 0.5, 0.9])
def test_full_size_tq1(N, p):
    """TQ1 at the sweep's shapes and every zero fraction of the workload, all
    output columns (M = 64 runs the tiled kernel at N = 8192, the skinny one
    with two activation slices at N = 28672)."""
    K = 8192
    T, s = iid_problem(N, K, p, 40)
    qd, sd = dev(pack("tq1", T)), dev(s)
    R = DenseRef(T, s)
    for M in (1, 4, 16, 64):
        say(f"[full tq1] N={N} p={p} M={M} {tq.tq_kernel_name(1, M, N, K)}")
        X = activations(M, K, 40 + M)
        Y = run("tq1", X, qd, sd, "auto").cpu().numpy()
        check_close(Y, R(X), f"full tq1 N={N} p={p} M={M}")


@pytest.mark.parametrize("path", ["auto", "skinny"])
def test_tq1_batch_rows_full_size(path):
    """TQ1 at 17..40 activation rows on N = K = 8192: the skinny kernel's
    two-slice template (a 32-row activation tile) with two row groups per
    workgroup, and the automatic choice there; every output column."""
    N = K = 8192
    T, s = iid_problem(N, K, 0.31, 48)
    qd, sd = dev(pack("tq1", T)), dev(s)
    R = DenseRef(T, s)
    for M in (17, 24, 32, 40):
        say(f"[tq1 batch] {path} M={M} {tq.tq_kernel_name(1, M, N, K, PATHS[path])}")
        X = activations(M, K, 48 + M)
        Y = run("tq1", X, qd, sd, path).cpu().numpy()
        check_close(Y, R(X), f"tq1 batch {path} M={M}")


def _overflow_problem(N, K):
    """Rows of X: +1000 everywhere, -1000 everywhere, 0.01 everywhere; weight
    rows all +1 (first half) or all -1 (second half), scale 1: the first two
    rows of Y are +-K * 1000 (past 65504: +-inf in fp16), the third +-K / 100."""
    X = np.zeros((3, K), np.float16)
    X[0], X[1], X[2] = 1000.0, -1000.0, 0.01
    T = np.ones((N, K), np.int8)
    T[N // 2:] = -1
    s = np.ones((N, K // 256), np.float16)
    return X, T, s


def _check_overflow(Y, X, T, s, label):
    want = ref(X, T, s)
    over = np.abs(want) > 65520.0  # rounds to +-inf in fp16 (nearest even)
    assert over[:2].all() and not over[2].any()
    Y64 = Y.astype(np.float64)
    assert np.array_equal(Y64[over], np.where(want[over] > 0, np.inf, -np.inf)), label
    check_close(Y[~over], want[~over], label)


@pytest.mark.parametrize("path", ["simple", "skinny", "tiled", "auto"])
@pytest.mark.parametrize("fmt", ["tq2", "tq1"])
def test_overflow_gives_inf(fmt, path):
    """An fp32 sum past the fp16 range becomes +-inf on every path (one
    round-to-nearest-even conversion), finite entries stay within the bound."""
    need(fmt, path)
    N, K = 96, 1280
    X, T, s = _overflow_problem(N, K)
    say(f"[overflow] {fmt} {path}")
    Y = run(fmt, X, pack(fmt, T), s, path).cpu().numpy()
    _check_overflow(Y, X, T, s, f"overflow {fmt}/{path}")


def test_overflow_gives_inf_other_entry_points():
    """The same through the tiled kernel at M > 16, the workspace product and
    the fused SwiGLU product (silu(g) u with g = u = 1.28e6 overflows too)."""
    from oracle import swiglu_ref
    N, K = 96, 1280
    X, T, s = _overflow_problem(N, K)
    X40 = np.concatenate([X, np.full((37, K), 0.01, np.float16)])
    T40, s40 = T, s
    Y = run("tq2", X40, pack("tq2", T40), s40, "auto").cpu().numpy()
    _check_overflow(Y[:3], X, T, s, "overflow tq2 M=40")
    ws = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda")
    Y = tq.tq_gemm_tq1_ws(dev(X40), dev(pack("tq1", T)), dev(s), ws).cpu().numpy()
    _check_overflow(Y[:3], X, T, s, "overflow tq1 ws M=40")
    Y = tq.tq_gemm_tq2_swiglu(dev(X), dev(pack("tq2", T)), dev(s), dev(pack("tq2", T)),
                              dev(s)).cpu().numpy()
    want = swiglu_ref(X, T, s, T, s)
    over = np.abs(want) > 65520.0
    # g = u = +1.28e6 overflows; g = u = -1.28e6 gives silu(g) u = -0 * u = +0
    assert over[0, :N // 2].all() and over[1, N // 2:].all() and not over[2].any()
    assert np.array_equal(Y.astype(np.float64)[over], np.where(want[over] > 0, np.inf, -np.inf))
    check_close(Y[~over], want[~over], "overflow swiglu")


def _wide_range_activations(M, K, seed):
    """Rows of fp16 subnormals (|x| < 2^-14) with one outlier channel of
    magnitude about 6e4 per row (at a different k in each row), and below
    them the same rows without the outlier."""
    rng = np.random.default_rng(seed)
    sub = (rng.integers(-1023, 1024, size=(M, K)) * 2.0 ** -24).astype(np.float16)
    out = sub.copy()
    ks = rng.integers(0, K, size=M)
    out[np.arange(M), ks] = rng.choice(np.array([60000.0, -60000.0, 59000.0]), size=M)
    return out, sub


@pytest.mark.parametrize("path", ["simple", "skinny", "tiled", "auto"])
@pytest.mark.parametrize("fmt", ["tq2", "tq1"])
def test_outlier_next_to_subnormal_activations(fmt, path):
    """Activations of the widest fp16 dynamic range: an outlier channel of
    about 6e4 among subnormal inputs (the skinny paths pre-scale staged
    activations by 1/4 and cancel the d' = d + 1 offset in fp32), and the
    subnormal rows alone, each call against the oracle within the bound."""
    need(fmt, path)
    K = 1536
    T, s = iid_problem(200, K, 0.31, 76)
    q = pack(fmt, T)
    for M in ((5, 16, 32) if fmt == "tq2" and path == "skinny" else (5, 16, 40)):
        Xo, Xs = _wide_range_activations(M, K, 77 + M)
        say(f"[wide range] {fmt} {path} M={M}")
        Y = run(fmt, Xo, q, s, path).cpu().numpy()
        check_close(Y, ref(Xo, T, s), f"outlier {fmt}/{path} M={M}")
        Y = run(fmt, Xs, q, s, path).cpu().numpy()
        check_close(Y, ref(Xs, T, s), f"subnormal {fmt}/{path} M={M}")


def test_outlier_activations_workspace_product():
    """The same wide-range activations through the TQ1 workspace product."""
    K, N, M = 1536, 200, 40
    T, s = iid_problem(N, K, 0.31, 78)
    Xo, Xs = _wide_range_activations(M, K, 79)
    ws = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda")
    for X, label in ((Xo, "outlier"), (Xs, "subnormal")):
        Y = tq.tq_gemm_tq1_ws(dev(X), dev(pack("tq1", T)), dev(s), ws).cpu().numpy()
        check_close(Y, ref(X, T, s), f"{label} tq1 ws")


# The seven linears of one layer of the 80-layer stack (K, N): q, k, v, o,
# gate, up, down.
STACK_LINEARS = {"q": (8192, 8192), "kv": (8192, 1024), "gate_up": (8192, 28672),
                 "down": (28672, 8192)}


@pytest.mark.parametrize("fmt", ["tq2", "tq1"])
@pytest.mark.parametrize("name", list(STACK_LINEARS))
def test_stack_layer_shapes(fmt, name):
    """Every distinct linear shape of the stack at M = 1 and 16 on the automatic
    kernel choice: every output column against the oracle."""
    K, N = STACK_LINEARS[name]
    T, s = iid_problem(N, K, 0.31, 90)
    q = pack(fmt, T)
    R = DenseRef(T, s)
    for M in (1, 16):
        say(f"[stack] {fmt} {name} M={M} K={K} N={N}")
        X = activations(M, K, 90 + M)
        Y = run(fmt, X, q, s, "auto").cpu().numpy()
        check_close(Y, R(X), f"stack {fmt} {name} M={M}")


PREFILL = [(256, 8192), (1024, 8192), (4096, 8192), (256, 28672)]


@pytest.mark.parametrize("fmt", ["tq2", "tq1"])
@pytest.mark.parametrize("M,N", PREFILL)
def test_prefill_sizes(fmt, M, N):
    """Prompt-sized products (K = 8192) on the automatic kernel choice: every
    row, and columns stratified over the whole width (one in every 16, both
    edges of every 32-column tile), against the oracle; all outputs finite."""
    K = 8192
    T, s = iid_problem(N, K, 0.31, 70)
    q = pack(fmt, T)
    cols = strat_cols(N, 71 + M)
    say(f"[prefill] {fmt} M={M} N={N} kernel={tq.tq_kernel_name(2 if fmt == 'tq2' else 1, M, N, K)}")
    X = activations(M, K, 70 + M)
    Y = run(fmt, X, q, s, "auto").cpu().numpy()
    assert np.all(np.isfinite(Y.astype(np.float32)))
    check_close(Y[:, cols], ref(X, T, s, cols=cols), f"prefill {fmt} M={M} N={N}")


# ---- fused decode-step linears

SWIGLU_SHAPES = [(1, 100, 256), (5, 300, 768), (16, 1000, 2048), (3, 4096, 8192),
                 (16, 1000, 6144)]


@pytest.mark.parametrize("M,N,K", SWIGLU_SHAPES)
def test_swiglu_parity(M, N, K):
    """Fused gate / up + SwiGLU against the fp64 oracle: ragged N, one to
    several row groups per workgroup, K with 1..32 blocks (the last in two
    activation windows)."""
    from oracle import swiglu_ref
    say(f"[swiglu] M={M} N={N} K={K}")
    Tg, sg = iid_problem(N, K, 0.31, 41)
    Tu, su = iid_problem(N, K, 0.31, 42)
    X = activations(M, K, 43)
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tq.tq_gemm_tq2_swiglu(dev(X), dev(pack("tq2", Tg)), dev(sg), dev(pack("tq2", Tu)), dev(su), Y)
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), swiglu_ref(X, Tg, sg, Tu, su), f"swiglu {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 16])
def test_swiglu_layer_shape(M):
    """The 70B gate / up shape (K = 8192, N = 28672): every output column
    against the oracle."""
    from oracle import swiglu_ref
    K, N = 8192, 28672
    say(f"[swiglu] layer M={M}")
    Tg, sg = iid_problem(N, K, 0.31, 44)
    Tu, su = iid_problem(N, K, 0.31, 45)
    X = activations(M, K, 46)
    Y = tq.tq_gemm_tq2_swiglu(dev(X), dev(pack("tq2", Tg)), dev(sg), dev(pack("tq2", Tu)),
                              dev(su)).cpu().numpy()
    check_close(Y, swiglu_ref(X, Tg, sg, Tu, su), f"swiglu layer M={M}")


def test_qkv_as_one_product():
    """q, k and v of a layer as one product over the row-concatenated packed
    matrices (N = 8192 + 1024 + 1024): one launch, and each slice of Y equals
    its own product against the oracle."""
    K = 8192
    parts = [(8192, 51), (1024, 52), (1024, 53)]
    Ts = [iid_problem(n, K, 0.31, sd) for n, sd in parts]
    T = np.concatenate([t for t, _ in Ts])
    s = np.concatenate([sc for _, sc in Ts])
    qs = pack("tq2", T)
    assert np.array_equal(qs, np.concatenate([pack("tq2", t) for t, _ in Ts]))
    for M in (1, 4):
        say(f"[qkv] M={M}")
        X = activations(M, K, 54 + M)
        Y = run("tq2", X, qs, s, "auto").cpu().numpy()
        check_close(Y, ref(X, T, s), f"qkv M={M}")
        n0 = 0
        for (t, sc), (n, _) in zip(Ts, parts):
            c = np.array([0, n // 2, n - 1])
            check_close(Y[:, n0 + c], ref(X, t, sc, cols=c), f"qkv slice {n} M={M}")
            n0 += n


# ---- QAT backward: input gradient through the ternary matrix

BWD_SHAPES = [(1, 8, 256), (5, 40, 512), (130, 264, 768), (257, 1000, 1280), (64, 2048, 8192)]


@pytest.mark.parametrize("M,N,K", BWD_SHAPES)
def test_bwd_x_parity(M, N, K):
    """dX = dY (s . T) against the fp64 oracle: ragged M (tiles of 128 rows),
    N in chunks of 32 with a ragged tail, K over several 128-column tiles."""
    from oracle import gemm_bwd_x_ref
    say(f"[bwd_x] M={M} N={N} K={K}")
    T, s = iid_problem(N, K, 0.31, 61)
    dY = activations(M, N, 62)
    dX = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    tq.tq_gemm_tq2_bwd_x(dev(dY), dev(pack("tq2", T)), dev(s), dX)
    torch.cuda.synchronize()
    check_close(dX.cpu().numpy(), gemm_bwd_x_ref(dY, T, s), f"bwd_x {M}x{N}x{K}")


def test_bwd_x_exact_integers():
    """Integer dY in [-3, 3] and scales in {1/4, 1/2, 1, 2}: every partial sum
    is exact in fp32, so dX must equal the oracle rounded once to fp16, value
    for value.  Two 512-row tiles (the second ragged) and a ragged last chunk
    of n."""
    from oracle import gemm_bwd_x_ref
    M, N, K = 520, 264, 768
    rng = np.random.default_rng(71)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    s = (2.0 ** rng.integers(-2, 2, size=(N, K // 256))).astype(np.float16)
    dY = rng.integers(-3, 4, size=(M, N)).astype(np.float16)
    say(f"[bwd_x exact] M={M} N={N} K={K}")
    dX = tq.tq_gemm_tq2_bwd_x(dev(dY), dev(pack("tq2", T)), dev(s)).cpu().numpy()
    ref = gemm_bwd_x_ref(dY, T, s).astype(np.float16)
    assert np.array_equal(dX.astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("kind", ["large", "subnormal"])
def test_bwd_x_scale_extremes(kind):
    """Scales near the documented bound (|s| = 1000: the kernel carries up to
    64 s in fp16) and fp16-subnormal scales (2^-20, 3 * 2^-24): finite and
    within the bound."""
    from oracle import gemm_bwd_x_ref
    M, N, K = 64, 96, 1024
    T, _ = iid_problem(N, K, 0.31, 72)
    rng = np.random.default_rng(73)
    if kind == "large":
        s = rng.choice(np.array([1000.0, -1000.0, 999.5, 512.0]), size=(N, K // 256))
        dY = rng.standard_normal((M, N)) * 0.01
    else:
        s = rng.choice(np.array([2.0 ** -20, 3 * 2.0 ** -24, -(2.0 ** -17)]), size=(N, K // 256))
        dY = rng.standard_normal((M, N)) * 100.0
    s, dY = s.astype(np.float16), dY.astype(np.float16)
    say(f"[bwd_x scales {kind}]")
    dX = tq.tq_gemm_tq2_bwd_x(dev(dY), dev(pack("tq2", T)), dev(s))
    torch.cuda.synchronize()
    check_close(dX.cpu().numpy(), gemm_bwd_x_ref(dY, T, s), f"bwd_x scales {kind}")


def test_bwd_x_full_size_sampled():
    """The bench's launch at full size, M = 4096 tokens, N = K = 8192: every
    row, and columns k stratified over the whole width (one in every 16, both
    edges of every 32-column tile, so both sides of every scale block and
    128-column tile) against the oracle."""
    from oracle import gemm_bwd_x_ref
    M, N, K = 4096, 8192, 8192
    T, s = iid_problem(N, K, 0.31, 74)
    dY = activations(M, N, 75)
    say(f"[bwd_x full] M={M} N={N} K={K}")
    dX = tq.tq_gemm_tq2_bwd_x(dev(dY), dev(pack("tq2", T)), dev(s))
    torch.cuda.synchronize()
    cols = strat_cols(K, 76)
    check_close(dX[:, cols].cpu().numpy(), gemm_bwd_x_ref(dY, T, s, cols=cols), "bwd_x full")


def test_bwd_x_adjoint_of_forward():
    """<Y, dY> = <X, dX> for Y from tq_gemm_tq2 and dX from the backward, both
    on the device (fp16 outputs, so within their rounding)."""
    M, N, K = 16, 512, 1024
    T, s = iid_problem(N, K, 0.31, 63)
    q = dev(pack("tq2", T))
    X, dY = activations(M, K, 64), activations(M, N, 65)
    Y = tq.tq_gemm_tq2(dev(X), q, dev(s)).cpu().numpy().astype(np.float64)
    dX = tq.tq_gemm_tq2_bwd_x(dev(dY), q, dev(s)).cpu().numpy().astype(np.float64)
    lhs, rhs = float(np.sum(Y * dY)), float(np.sum(X.astype(np.float64) * dX))
    scale = float(np.sum(np.abs(Y * dY)))
    assert abs(lhs - rhs) <= 2e-3 * scale, (lhs, rhs, scale)


# ---- TQ1 -> TQ2 transcoding and the TQ1 product with a workspace

@pytest.mark.parametrize("N,K,ldq", [(1, 256, None), (37, 768, None), (100, 1280, 272),
                                     (513, 8192, None)])
def test_transcode_matches_host_packer(N, K, ldq):
    """Device re-packing of TQ1 bytes equals the host TQ2 packing of the same
    trits, byte for byte (ragged units at the row end, a padded ldq)."""
    T, _ = iid_problem(N, K, 0.31, 91)
    q1 = pack("tq1", T) if ldq is None else pack_tq1_ref(T, ldq)
    say(f"[transcode] N={N} K={K} ldq={q1.shape[1]}")
    q2 = tq.tq_transcode_tq1_tq2(dev(q1), K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q2.cpu().numpy(), pack("tq2", T))


@pytest.mark.parametrize("M,N", [(16, 200), (17, 200), (95, 200), (96, 200), (130, 200),
                                 (32, 16392), (33, 16392)])
def test_gemm_tq1_ws(M, N):
    """From tq_tq1_transcode_min_m(N, K) rows on the workspace product equals
    tq_gemm_tq2 on the same trits bit for bit; below, it equals tq_gemm_tq1;
    both match the oracle (both sides of both switch points)."""
    K = 1024
    T, s = iid_problem(N, K, 0.31, 92)
    X = activations(M, K, 93)
    ws = torch.empty(N * K // 4 + 64, dtype=torch.uint8, device="cuda")
    say(f"[tq1 ws] M={M} N={N}")
    Y = tq.tq_gemm_tq1_ws(dev(X), dev(pack("tq1", T)), dev(s), ws).cpu().numpy()
    if M >= tq.tq_tq1_transcode_min_m(N, K):
        Y2 = tq.tq_gemm_tq2(dev(X), dev(pack("tq2", T)), dev(s)).cpu().numpy()
    else:
        Y2 = tq.tq_gemm_tq1(dev(X), dev(pack("tq1", T)), dev(s)).cpu().numpy()
    np.testing.assert_array_equal(Y.view(np.uint16), Y2.view(np.uint16))
    check_close(Y, ref(X, T, s), f"tq1 ws M={M} N={N}")


def test_gemm_tq1_ws_small_workspace_runs_tq1():
    """A workspace smaller than N * K / 4 bytes is not used: the TQ1 kernels run."""
    M, N, K = 64, 96, 512
    T, s = iid_problem(N, K, 0.31, 94)
    X = activations(M, K, 95)
    ws = torch.full((N * K // 4 - 16,), 0xAB, dtype=torch.uint8, device="cuda")
    Y = tq.tq_gemm_tq1_ws(dev(X), dev(pack("tq1", T)), dev(s), ws).cpu().numpy()
    Y1 = tq.tq_gemm_tq1(dev(X), dev(pack("tq1", T)), dev(s)).cpu().numpy()
    np.testing.assert_array_equal(Y.view(np.uint16), Y1.view(np.uint16))
    assert bool((ws == 0xAB).all())


@pytest.mark.parametrize("M,N", [(64, 28672), (256, 8192)])
def test_gemm_tq1_ws_full_size(M, N):
    """The sweep's TQ1 batch point and a prefill size through the workspace
    path, every output column against the oracle."""
    K = 8192
    T, s = iid_problem(N, K, 0.3, 96)
    X = activations(M, K, 97)
    ws = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda")
    say(f"[tq1 ws full] M={M} N={N}")
    Y = tq.tq_gemm_tq1_ws(dev(X), dev(pack("tq1", T)), dev(s), ws)
    torch.cuda.synchronize()
    check_close(Y.cpu().numpy(), DenseRef(T, s)(X), f"tq1 ws full M={M} N={N}")


def test_stream_read_covers_every_piece():
    """The read-ceiling kernel folds every 16-byte piece: a lone piece whose
    dwords XOR to the marker is found wherever it sits; zeros write nothing."""
    marker = 0x9E3779B9 - (1 << 32)  # as int32
    n = (1 << 20) + 48  # not a multiple of the pieces one pass of the grid reads
    src = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    tq.tq_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 7
    for piece in (0, 1, 4095, n // 32, n // 16 - 1):
        src.zero_()
        src[4 * piece] = marker
        sink.fill_(7)
        tq.tq_stream_read(src, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) == marker, piece


def test_empty_is_noop():
    X = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    q = torch.empty((16, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((16, 1), dtype=torch.float16, device="cuda")
    Y = tq.tq_gemm_tq2(X, q, s)
    assert Y.shape == (0, 16)


_CONCURRENT_FIRST_CALLS = r"""
import sys, threading
import numpy as np
import torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + '/tests')
import bit_mixed_precision_amd.binding as tq
from gpu_util import activations, iid_problem, check_close, ref
torch.cuda.set_device(0)
N, K = 512, 8192
T, s = iid_problem(N, K, 0.31, 88)
q2, q1 = tq.tq_pack_tq2(T)[0], tq.tq_pack_tq1(T)[0]
calls = [("tq2", 8), ("tq2", 128), ("tq1", 8), ("tq1", 64)]
inputs = {c: activations(c[1], K, 88 + c[1]) for c in calls}
dev = {k: torch.from_numpy(v).cuda() for k, v in {"q2": q2, "q1": q1, "s": s}.items()}
X = {c: torch.from_numpy(x).cuda() for c, x in inputs.items()}
torch.cuda.synchronize()
start = threading.Barrier(2)
out, errs = {}, []
def work(t):
    try:
        torch.cuda.set_device(0)
        start.wait()
        for fmt, M in calls:  # first calls of kernels whose LDS exceeds 64 KB
            fn = tq.tq_gemm_tq2 if fmt == "tq2" else tq.tq_gemm_tq1
            out[(t, fmt, M)] = fn(X[(fmt, M)], dev["q2" if fmt == "tq2" else "q1"], dev["s"])
        torch.cuda.synchronize()
    except Exception as e:  # reported by the main thread
        errs.append(repr(e))
th = [threading.Thread(target=work, args=(t,)) for t in range(2)]
[x.start() for x in th]; [x.join() for x in th]
assert not errs, errs
for fmt, M in calls:
    a, b = out[(0, fmt, M)].cpu().numpy(), out[(1, fmt, M)].cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (fmt, M)
    check_close(a, ref(inputs[(fmt, M)], T, s), f"{fmt} M={M}")
print("CONCURRENT-OK", flush=True)
"""


def test_concurrent_first_calls_from_two_threads():
    """Two host threads make the first calls of every large-LDS kernel family
    at the same time, in a fresh process (the per-device attribute set-up is
    shared state): both succeed and give the same bits, matching the oracle."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("[concurrent first calls] subprocess")
    out = subprocess.run([sys.executable, "-c", _CONCURRENT_FIRST_CALLS, root],
                         capture_output=True, text=True, timeout=110)
    assert "CONCURRENT-OK" in out.stdout, out.stdout[-2000:] + out.stderr[-2000:]
