"""libtq.so loads, exports every symbol include/tq.h declares, and rejects bad
arguments with the documented codes before touching memory (CPU only)."""

import ctypes as C
import os
import re
import subprocess
import sys

import pytest

tq = pytest.importorskip("bit_mixed_precision_amd.binding")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")
HAS_GPU = os.path.exists("/dev/kfd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", tq._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (tq_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    assert set(names) == set(tq.SIGNATURES)
    for n in names:
        assert hasattr(tq.lib, n)


def test_status_and_sizes():
    assert tq.tq_abi_version() == 1
    assert tq.tq_status_string(0) == "ok"
    assert tq.tq_status_string(-4).startswith("pointer")
    assert tq.tq_status_string(123) == "unknown status"
    assert tq.tq_tq2_bytes(8192, 8192) == 16777216
    assert tq.tq_tq2_bytes(8192, 28672) * 1 == 58720256
    assert tq.tq_num_scales(8192, 8192) * 2 == 524288
    assert tq.tq_tq1_ldq(8192) == 1648 and tq.tq_tq1_ldq(1024) == 208
    assert tq.tq_tq2_bytes(-1, 4) == -1 and tq.tq_num_scales(1, 100) == -1


A = 0x10000  # a 16-byte aligned fake address: never dereferenced by the checks below


def _g2(X=A, q=A, s=A, Y=A, M=1, N=16, K=256, path=0):
    return tq.raw_call("tq_gemm_tq2_ex", X, q, s, Y, M, N, K, path, None)


def _g1(X=A, q=A, ldq=64, s=A, Y=A, M=1, N=16, K=256, path=0):
    return tq.raw_call("tq_gemm_tq1_ex", X, q, ldq, s, Y, M, N, K, path, None)


def test_gemm_argument_errors():
    # null -> shape -> alignment -> value, each before any device work
    assert _g2(X=None) == tq.TQ_ERR_NULL
    assert _g2(Y=None, K=100) == tq.TQ_ERR_NULL
    assert _g2(K=100) == tq.TQ_ERR_SHAPE
    assert _g2(K=0) == tq.TQ_ERR_SHAPE
    assert _g2(M=-1) == tq.TQ_ERR_SHAPE
    assert _g2(M=(1 << 24) + 1) == tq.TQ_ERR_SHAPE
    assert _g2(K=(1 << 20) + 256) == tq.TQ_ERR_SHAPE
    assert _g2(X=A + 8, K=100) == tq.TQ_ERR_SHAPE
    assert _g2(X=A + 8) == tq.TQ_ERR_ALIGN
    assert _g2(s=A + 2) == tq.TQ_ERR_ALIGN
    assert _g2(path=9) == tq.TQ_ERR_VALUE
    assert _g1(ldq=51) == tq.TQ_ERR_SHAPE      # < ceil(256/5)
    assert _g1(ldq=56) == tq.TQ_ERR_SHAPE      # not a multiple of 16
    assert _g1(q=A + 4) == tq.TQ_ERR_ALIGN
    # empty products are no-ops that touch no pointer
    assert _g2(X=None, q=None, s=None, Y=None, M=0) == tq.TQ_OK
    assert _g1(X=None, q=None, s=None, Y=None, N=0) == tq.TQ_OK
    assert tq.raw_call("tq_gemm_tq2", None, None, None, None, 0, 5, 256, None) == tq.TQ_OK


def _gt(mt, ng, kg, X=A, M=40, K=512):
    return tq.raw_call("tq_gemm_tq2_tiled", X, A, A, A, M, 64, K, mt, ng, kg, None)


def test_tiled_tile_errors():
    # argument checks first, then the tile, both before any device work
    assert _gt(4, 2, 2, X=None) == tq.TQ_ERR_NULL
    assert _gt(4, 2, 2, K=300) == tq.TQ_ERR_SHAPE
    for tile in [(3, 2, 2), (4, 4, 4), (4, 1, 8), (2, 2, 8), (4, 8, 1), (0, 2, 2), (4, 1, 2)]:
        assert _gt(*tile) == tq.TQ_ERR_UNSUPPORTED, tile
    assert _gt(3, 2, 2, X=None, M=0) == tq.TQ_OK


def _gt4(mt, nr, ng, kg, X=A, M=40, K=512):
    return tq.raw_call("tq_gemm_tq2_tile", X, A, A, A, M, 64, K, mt, nr, ng, kg, None)


def test_tile_errors():
    assert _gt4(2, 2, 1, 4, X=None) == tq.TQ_ERR_NULL
    assert _gt4(2, 2, 1, 4, K=300) == tq.TQ_ERR_SHAPE
    for tile in [(2, 2, 4, 2), (2, 2, 2, 2), (2, 3, 1, 4), (8, 4, 4, 2), (4, 1, 1, 4),
                 (3, 2, 1, 4), (4, 2, 1, 8), (4, 4, 1, 8), (2, 4, 2, 8)]:
        assert _gt4(*tile) == tq.TQ_ERR_UNSUPPORTED, tile
    assert _gt4(3, 2, 1, 4, X=None, M=0) == tq.TQ_OK


def _gt1(mt, nr, ng, kg, X=A, M=40, K=512, ldq=112):
    return tq.raw_call("tq_gemm_tq1_tile", X, A, ldq, A, A, M, 64, K, mt, nr, ng, kg, None)


def test_tq1_tile_errors():
    # argument checks, then the tile and the table kernel's row-stride limit,
    # all before any device work
    assert _gt1(2, 2, 1, 4, X=None) == tq.TQ_ERR_NULL
    assert _gt1(2, 2, 1, 4, K=300) == tq.TQ_ERR_SHAPE
    assert _gt1(2, 2, 1, 4, ldq=96) == tq.TQ_ERR_SHAPE  # < ceil(512/5)
    for tile in [(2, 2, 4, 2), (2, 2, 2, 2), (2, 3, 1, 4), (8, 4, 4, 2), (4, 1, 1, 4),
                 (3, 2, 1, 4), (4, 2, 1, 8), (4, 4, 1, 8), (2, 4, 2, 8)]:
        assert _gt1(*tile) == tq.TQ_ERR_UNSUPPORTED, tile
    assert _gt1(2, 2, 1, 4, ldq=(1 << 22) + 16) == tq.TQ_ERR_UNSUPPORTED
    assert _gt1(3, 2, 1, 4, X=None, M=0) == tq.TQ_OK


def test_pack_dev_argument_errors():
    wsb = tq.lib.tq_pack_dev_workspace_bytes(64, 512)
    assert wsb > 256 * 8
    assert tq.lib.tq_pack_dev_workspace_bytes(0, 512) == -1
    assert tq.lib.tq_pack_dev_workspace_bytes(4, 300) == -1

    def p2(W=A, N=64, K=512, q=A, s=A, ws=A, wsb=wsb):
        return tq.raw_call("tq_pack_tq2_dev", W, N, K, 1e-5, q, s, None, None, ws, wsb, None)

    assert p2(W=None) == tq.TQ_ERR_NULL
    assert p2(ws=None) == tq.TQ_ERR_NULL
    assert p2(K=300) == tq.TQ_ERR_SHAPE
    assert p2(wsb=wsb - 8) == tq.TQ_ERR_SHAPE
    assert p2(W=A + 4) == tq.TQ_ERR_ALIGN
    assert tq.raw_call("tq_pack_tq1_dev", A, 64, 512, 1e-5, 96, A, A, None, None, A, wsb,
                       None) == tq.TQ_ERR_SHAPE  # ldq < ceil(512 / 5)


@pytest.mark.skipif(HAS_GPU, reason="checks the no-device error; a GPU is present")
def test_gemm_without_device():
    assert _g2() == tq.TQ_ERR_DEVICE
    assert _g1() == tq.TQ_ERR_DEVICE
    assert tq.raw_call("tq_gemm_tq2", A, A, A, A, 4, 32, 512, None) == tq.TQ_ERR_DEVICE


def test_host_argument_errors():
    P = C.c_void_p
    buf = (C.c_uint8 * 4096)()
    assert tq.raw_call("tq_pack_tq2", 0, None, 1, 256, 0.0, buf, None, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_pack_tq2", 1, buf, 1, 256, 0.0, buf, None, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_pack_tq2", 5, buf, 1, 256, 0.0, buf, buf, None) == tq.TQ_ERR_VALUE
    assert tq.raw_call("tq_pack_tq2", 0, buf, 0, 256, 0.0, buf, None, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_pack_tq1", 0, buf, 1, 256, 0.0, 10, buf, None, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_unpack_tq2", None, 1, 4, buf) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_unpack_tq2", buf, 1, 6, buf) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_unpack_tq1", buf, 1, 5, 0, buf) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_ternarize_f32", None, 1, 1, 0.0, None, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_ternarize_f32", P(C.addressof(buf)), 0, 1, 0.0, None, None) == tq.TQ_ERR_SHAPE


def test_package_fails_loudly_without_library(tmp_path):
    """A copy of the package without libtq.so raises ImportError on use."""
    import shutil
    pkg = tmp_path / "bit_mixed_precision_amd"
    shutil.copytree(os.path.join(ROOT, "bit_mixed_precision_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    code = ("import bit_mixed_precision_amd as b\n"
            "try:\n    b.tq_gemm_tq2\nexcept ImportError as e:\n    print('IMPORT-ERROR', e)\n")
    env = {k: v for k, v in os.environ.items() if k != "TQ_LIBRARY"}  # the default path only
    out = subprocess.run(["python", "-c", code], cwd=tmp_path, capture_output=True, text=True,
                         env=env)
    assert "IMPORT-ERROR" in out.stdout, out.stdout + out.stderr


def test_one_hip_runtime_per_process():
    """Importing the binding before torch must not map a second HIP runtime:
    libtq.so and the torch wheel both need libamdhip64.so.7, and two copies in
    one process crash on the first device allocation."""
    pytest.importorskip("torch")
    code = ("import bit_mixed_precision_amd.binding\nimport torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps')\n"
            "         if 'libamdhip64' in l or 'libhsa-runtime64' in l}\n"
            "print(len([p for p in paths if 'amdhip64' in p]),"
            " len([p for p in paths if 'hsa-runtime64' in p]))\n")
    out = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.split()
    assert out == ["1", "1"], out


def _sg(X=A, gate=A, up=A, M=4, N=64, K=512, Y=A):
    return tq.raw_call("tq_gemm_tq2_swiglu", X, gate, A, up, A, Y, M, N, K, None)


def test_swiglu_argument_errors():
    """Checks in order: shape of M, N, then null, shape of K, alignment, then
    the decode-size limit (M <= 16), all before any device work."""
    assert _sg(M=0, X=None) == tq.TQ_OK
    assert _sg(N=0, up=None) == tq.TQ_OK
    assert _sg(M=-1) == tq.TQ_ERR_SHAPE
    assert _sg(X=None) == tq.TQ_ERR_NULL
    assert _sg(gate=None) == tq.TQ_ERR_NULL
    assert _sg(up=None) == tq.TQ_ERR_NULL
    assert _sg(K=300) == tq.TQ_ERR_SHAPE
    assert _sg(up=A + 2) == tq.TQ_ERR_ALIGN
    assert _sg(M=17) == tq.TQ_ERR_UNSUPPORTED


def test_build_step_does_not_load_the_library():
    """Resolving the build module must not load libtq.so (a library loaded
    before a rebuild stays mapped, and the fresh symbols would be missing)."""
    code = ("import sys; sys.path.insert(0, %r); "
            "from bit_mixed_precision_amd import build_lib; "
            "import bit_mixed_precision_amd.build_lib; "
            "print('bit_mixed_precision_amd.binding' in sys.modules)") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "False"


def _bx(dY=A, q=A, s=A, dX=A, M=4, N=64, K=512):
    return tq.raw_call("tq_gemm_tq2_bwd_x", dY, q, s, dX, M, N, K, None)


def test_bwd_x_argument_errors():
    assert _bx(M=0, dY=None) == tq.TQ_OK
    assert _bx(M=-1) == tq.TQ_ERR_SHAPE
    assert _bx(dX=None) == tq.TQ_ERR_NULL
    assert _bx(q=None) == tq.TQ_ERR_NULL
    assert _bx(N=0) == tq.TQ_ERR_SHAPE
    assert _bx(N=60) == tq.TQ_ERR_SHAPE
    assert _bx(N=(1 << 20) + 8) == tq.TQ_ERR_SHAPE  # past the 32-bit offsets of 512 rows
    assert _bx(K=300) == tq.TQ_ERR_SHAPE
    assert _bx(dY=A + 8) == tq.TQ_ERR_ALIGN


def test_stream_read_argument_errors():
    assert tq.raw_call("tq_stream_read", A, 0, A, None) == tq.TQ_OK
    assert tq.raw_call("tq_stream_read", A, -16, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_stream_read", A, 40, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_stream_read", None, 64, A, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_stream_read", A, 64, None, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_stream_read", A + 4, 64, A, None) == tq.TQ_ERR_ALIGN


def test_transcode_argument_errors():
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1648, 0, 8192, A, None) == tq.TQ_OK
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1648, -1, 8192, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_transcode_tq1_tq2", None, 1648, 4, 8192, A, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1648, 4, 8192, None, None) == tq.TQ_ERR_NULL
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1632, 4, 8192, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1650, 4, 8192, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1648, 4, 8000, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_transcode_tq1_tq2", A + 4, 1648, 4, 8192, A, None) == tq.TQ_ERR_ALIGN
    assert tq.raw_call("tq_transcode_tq1_tq2", A, 1648, 4, 8192, A + 8, None) == tq.TQ_ERR_ALIGN


def test_gemm_tq1_ws_argument_errors():
    assert tq.tq_tq1_transcode_min_m(8192, 8192) == 96
    assert tq.tq_tq1_transcode_min_m(28672, 8192) == 33
    assert tq.raw_call("tq_tq1_transcode_min_m", 0, 8192) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_tq1_transcode_min_m", 16, 300) == tq.TQ_ERR_SHAPE
    call = lambda ws=A, nb=1 << 20, M=64, X=A: tq.raw_call(
        "tq_gemm_tq1_ws", X, A, 64, A, A, M, 16, 256, ws, nb, None)
    assert call(M=0, X=None) == tq.TQ_OK
    assert call(X=None) == tq.TQ_ERR_NULL
    assert call(nb=-1) == tq.TQ_ERR_SHAPE
    assert call(ws=A + 4) == tq.TQ_ERR_ALIGN


def test_ldq_upper_bound():
    """The TQ1 kernels take ldq as a 32-bit int: strides past 2^24 are refused
    before any device work (else row offsets could wrap)."""
    big = (1 << 24) + 16
    assert _g1(ldq=big) == tq.TQ_ERR_SHAPE
    assert _g1(ldq=1 << 31) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_gemm_tq1_tile", A, A, big, A, A, 40, 64, 512, 2, 2, 1, 4,
                       None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_transcode_tq1_tq2", A, big, 4, 8192, A, None) == tq.TQ_ERR_SHAPE
    assert tq.raw_call("tq_gemm_tq1_ws", A, A, big, A, A, 64, 16, 256, A, 1 << 20,
                       None) == tq.TQ_ERR_SHAPE


# ---- the Python binding's checks of its tensor arguments (no device needed:
# every check but the last, the device, runs on CPU tensors)

def _t(shape, dtype):
    torch = pytest.importorskip("torch")
    return torch.zeros(shape, dtype=getattr(torch, dtype))


def _raises(status, fn, *a, **kw):
    with pytest.raises(tq.TQError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)


def test_binding_rejects_bad_gemm_tensors():
    X, q, s = _t((4, 512), "float16"), _t((32, 128), "uint8"), _t((32, 2), "float16")
    # well-formed CPU tensors get as far as the device check
    _raises(tq.TQ_ERR_DEVICE, tq.tq_gemm_tq2, X, q, s)
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq2, X.float(), q, s)
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq2, X, q.int(), s)
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq2, X, q, s.float())
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X, _t((32, 64), "uint8"), s)    # qs too short
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X, q, _t((32, 1), "float16"))  # scales too short
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X, q, _t((31, 2), "float16"))
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X.t(), q, s)                   # transposed X
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, _t((512, 4), "float16").t(), q, s)  # not contiguous
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X[0], q, s)                    # not 2-D
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2, X, q, s, _t((4, 31), "float16"))   # short Y
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq2, X, q, s, _t((4, 32), "float32"))   # wrong Y dtype
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_tile, X, q, _t((32, 1), "float16"), 2, 2, 1, 4)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_tiled, X, _t((16, 128), "uint8"), s, 2, 1, 4)
    # TQ1: qs [N][ldq]; scales still [N][K/256]
    q1 = _t((32, 112), "uint8")
    _raises(tq.TQ_ERR_DEVICE, tq.tq_gemm_tq1, X, q1, s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq1, X, q1, _t((32, 4), "float16"))
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq1, X, q1.half(), s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq1_tile, X, q1, _t((16, 2), "float16"), 2, 2, 1, 4)
    _raises(tq.TQ_ERR_DEVICE, tq.tq_gemm_tq1_ws, X, q1, s, _t((32 * 128,), "uint8"))
    _raises(tq.TQ_ERR_VALUE, tq.tq_gemm_tq1_ws, X, q1, s, _t((32 * 128,), "int32"))


def test_binding_rejects_bad_other_tensors():
    X, q, s = _t((4, 512), "float16"), _t((32, 128), "uint8"), _t((32, 2), "float16")
    _raises(tq.TQ_ERR_DEVICE, tq.tq_gemm_tq2_swiglu, X, q, s, q, s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_swiglu, X, q, s, _t((16, 128), "uint8"), s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_swiglu, X, q, s, q, _t((32, 1), "float16"))
    dY = _t((4, 32), "float16")
    _raises(tq.TQ_ERR_DEVICE, tq.tq_gemm_tq2_bwd_x, dY, q, s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_bwd_x, _t((4, 16), "float16"), q, s)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_gemm_tq2_bwd_x, dY, q, s, _t((4, 256), "float16"))
    _raises(tq.TQ_ERR_SHAPE, tq.tq_transcode_tq1_tq2, _t((32, 112), "uint8"), 512,
            _t((32, 64), "uint8"))
    _raises(tq.TQ_ERR_DEVICE, tq.tq_transcode_tq1_tq2, _t((32, 112), "uint8"), 512)
    _raises(tq.TQ_ERR_VALUE, tq.tq_pack_dev, 2, _t((32, 512), "float16"))
    _raises(tq.TQ_ERR_DEVICE, tq.tq_pack_dev, 2, _t((32, 512), "float32"))
    _raises(tq.TQ_ERR_VALUE, tq.tq_stream_read, _t((64,), "uint8"), _t((4,), "float32"))
    _raises(tq.TQ_ERR_DEVICE, tq.tq_stream_read, _t((64,), "uint8"), _t((4,), "int32"))


def _sg_w(dY=A, X=A, dW=A, M=64, N=64, K=64, acc=0):
    return tq.raw_call("tq_ste_grad_w", dY, X, dW, M, N, K, acc, None)


def test_ste_grad_w_argument_errors():
    """Shape, null, alignment and value checks before any device work; the
    documented no-ops touch no pointer."""
    assert _sg_w(dY=None, X=None, dW=None, N=0) == tq.TQ_OK
    assert _sg_w(dY=None, X=None, dW=None, K=0) == tq.TQ_OK
    assert _sg_w(dY=None, X=None, dW=None, M=0, acc=1) == tq.TQ_OK
    assert _sg_w(M=-1) == tq.TQ_ERR_SHAPE
    assert _sg_w(dW=None) == tq.TQ_ERR_NULL
    assert _sg_w(X=None) == tq.TQ_ERR_NULL
    assert _sg_w(dY=None, X=None, M=0, K=300) == tq.TQ_ERR_SHAPE  # M = 0 needs no inputs
    assert _sg_w(N=60) == tq.TQ_ERR_SHAPE
    assert _sg_w(K=12) == tq.TQ_ERR_SHAPE
    assert _sg_w(M=1 << 20, N=2048) == tq.TQ_ERR_SHAPE   # M N past 2^30
    assert _sg_w(M=1 << 20, K=2048) == tq.TQ_ERR_SHAPE
    assert _sg_w(N=(1 << 24) + 8, M=1) == tq.TQ_ERR_SHAPE
    assert _sg_w(X=A + 8) == tq.TQ_ERR_ALIGN
    assert _sg_w(dW=A + 4) == tq.TQ_ERR_ALIGN
    assert _sg_w(acc=2) == tq.TQ_ERR_VALUE


def test_binding_rejects_bad_ste_tensors():
    dY, X = _t((8, 64), "float16"), _t((8, 128), "float16")
    _raises(tq.TQ_ERR_DEVICE, tq.tq_ste_grad_w, dY, X)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_ste_grad_w, dY, _t((9, 128), "float16"))
    _raises(tq.TQ_ERR_VALUE, tq.tq_ste_grad_w, dY.float(), X)
    _raises(tq.TQ_ERR_SHAPE, tq.tq_ste_grad_w, dY, X, _t((64, 64), "float32"))
    _raises(tq.TQ_ERR_VALUE, tq.tq_ste_grad_w, dY, X, _t((64, 128), "float16"))
    _raises(tq.TQ_ERR_NULL, tq.tq_ste_grad_w, dY, X, None, True)
