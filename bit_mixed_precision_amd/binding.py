"""Python binding of libtq.so: the C entry points under the same names.

Argument marshalling only.  Host functions take numpy arrays; device functions
take torch tensors that already live on the GPU and pass their data pointers
and the current HIP stream.  Every status other than TQ_OK raises ``TQError``.
Importing this module raises ``ImportError`` when libtq.so has not been built:
there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

# One HIP runtime per process.  libtq.so needs libamdhip64.so.7, and the torch
# wheel carries its own copy of that library (and of the HSA runtime).  If
# libtq.so were loaded first, the system copy would be mapped and torch would
# then map its own: two runtimes claiming one GPU, which crashes on the first
# device allocation.  Importing torch first lets the loader resolve libtq.so's
# dependency to the copy torch already mapped.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # host-only use without torch: the system runtime is the only one
    _torch = None

# TQ_LIBRARY names another build of the same library (the sanitizer variant
# of build_lib); by default the in-tree libtq.so next to this file.
_LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libtq.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing; build it with "
                      "`python -m bit_mixed_precision_amd.build_lib`")
lib = C.CDLL(_LIB_PATH)

TQ_OK, TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_ERR_VALUE, TQ_ERR_ALIGN, TQ_ERR_DEVICE, TQ_ERR_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
TQ_SRC_TERNARY_I8, TQ_SRC_LATENT_F32 = 0, 1
TQ_PATH_AUTO, TQ_PATH_SKINNY, TQ_PATH_TILED, TQ_PATH_SIMPLE = 0, 1, 2, 3

_P, _I64, _I, _D = C.c_void_p, C.c_int64, C.c_int, C.c_double

#: Every symbol include/tq.h declares, with (restype, argtypes).
SIGNATURES = {
    "tq_status_string": (C.c_char_p, [_I]),
    "tq_abi_version": (_I, []),
    "tq_tq2_bytes": (_I64, [_I64, _I64]),
    "tq_tq1_ldq": (_I64, [_I64]),
    "tq_num_scales": (_I64, [_I64, _I64]),
    "tq_ternarize_f32": (_I, [_P, _I64, _I64, _D, _P, _P]),
    "tq_pack_tq2": (_I, [_I, _P, _I64, _I64, _D, _P, _P, _P]),
    "tq_pack_tq1": (_I, [_I, _P, _I64, _I64, _D, _I64, _P, _P, _P]),
    "tq_unpack_tq2": (_I, [_P, _I64, _I64, _P]),
    "tq_unpack_tq1": (_I, [_P, _I64, _I64, _I64, _P]),
    "tq_gemm_tq2": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "tq_gemm_tq1": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _I64, _P]),
    "tq_kernel_name": (_I, [_I, _I64, _I64, _I64, _I, C.c_char_p, _I64]),
    "tq_gemm_tq2_ex": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "tq_gemm_tq1_ex": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _I64, _I, _P]),
    "tq_gemm_tq2_tiled": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P]),
    "tq_gemm_tq2_tile": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P]),
    "tq_gemm_tq2_wide": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P]),
    "tq_gemm_tq2_swiglu": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "tq_gemm_tq2_bwd_x": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "tq_stream_read": (_I, [_P, _I64, _P, _P]),
    "tq_ste_grad_w": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "tq_transcode_tq1_tq2": (_I, [_P, _I64, _I64, _I64, _P, _P]),
    "tq_tq1_transcode_min_m": (_I64, [_I64, _I64]),
    "tq_gemm_tq1_ws": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "tq_gemm_tq1_tile": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P]),
    "tq_pack_dev_workspace_bytes": (_I64, [_I64, _I64]),
    "tq_pack_tq2_dev": (_I, [_P, _I64, _I64, C.c_double, _P, _P, _P, _P, _P, _I64, _P]),
    "tq_pack_tq1_dev": (_I, [_P, _I64, _I64, C.c_double, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "tq_pack_tq2_dev_noalloc": (_I, [_P, _I64, _I64, C.c_double, _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tq_status_string(status)} ({status})")


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


def _ptr(a) -> int | None:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()  # torch tensor


def tq_status_string(status: int) -> str:
    return lib.tq_status_string(status).decode()


def tq_abi_version() -> int:
    return lib.tq_abi_version()


def tq_tq2_bytes(N: int, K: int) -> int:
    return lib.tq_tq2_bytes(N, K)


def tq_tq1_ldq(K: int) -> int:
    return lib.tq_tq1_ldq(K)


def tq_num_scales(N: int, K: int) -> int:
    return lib.tq_num_scales(N, K)


# ------------------------------------------------------------------ host

def tq_ternarize_f32(W: np.ndarray, eps: float = 1e-5):
    """(T int8 [N][K], gamma) for float32 latents W [N][K]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    g = C.c_double(0.0)
    _check(lib.tq_ternarize_f32(_ptr(W), N, K, float(eps), _ptr(T), C.byref(g)), "tq_ternarize_f32")
    return T, g.value


def _src(W):
    W = np.asarray(W)
    if W.dtype == np.int8:
        return TQ_SRC_TERNARY_I8, np.ascontiguousarray(W)
    if W.dtype == np.float32:
        return TQ_SRC_LATENT_F32, np.ascontiguousarray(W)
    raise TypeError("W must be int8 trits or float32 latents")


def tq_pack_tq2(W: np.ndarray, eps: float = 1e-5):
    """Pack int8 trits or float32 latents W [N][K].

    Returns (qs uint8 [N][K/4], scales fp16 [N][K/256] or None, gamma or None);
    scales and gamma come back only for latents (fp16(gamma) in every block).
    """
    kind, W = _src(W)
    N, K = W.shape
    qs = np.empty((N, max(K // 4, 0)), dtype=np.uint8)
    scales = np.empty((N, max(K // 256, 0)), dtype=np.float16) if kind == TQ_SRC_LATENT_F32 else None
    g = C.c_double(0.0)
    _check(lib.tq_pack_tq2(kind, _ptr(W), N, K, float(eps), _ptr(qs), _ptr(scales), C.byref(g)),
           "tq_pack_tq2")
    return qs, scales, (g.value if scales is not None else None)


def tq_pack_tq1(W: np.ndarray, eps: float = 1e-5, ldq: int | None = None):
    """Like tq_pack_tq2 with the 1.6-bit packing; qs is uint8 [N][ldq]."""
    kind, W = _src(W)
    N, K = W.shape
    if ldq is None:
        ldq = tq_tq1_ldq(K)
    qs = np.empty((N, max(ldq, 0)), dtype=np.uint8)
    scales = np.empty((N, max(K // 256, 0)), dtype=np.float16) if kind == TQ_SRC_LATENT_F32 else None
    g = C.c_double(0.0)
    _check(lib.tq_pack_tq1(kind, _ptr(W), N, K, float(eps), ldq, _ptr(qs), _ptr(scales),
                           C.byref(g)), "tq_pack_tq1")
    return qs, scales, (g.value if scales is not None else None)


def tq_unpack_tq2(qs: np.ndarray, K: int) -> np.ndarray:
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    N = qs.shape[0]
    if qs.shape[1] * 4 != K:
        raise ValueError("qs does not hold K/4 bytes per row")
    T = np.empty((N, K), dtype=np.int8)
    _check(lib.tq_unpack_tq2(_ptr(qs), N, K, _ptr(T)), "tq_unpack_tq2")
    return T


def tq_unpack_tq1(qs: np.ndarray, K: int) -> np.ndarray:
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    N, ldq = qs.shape
    T = np.empty((N, K), dtype=np.int8)
    _check(lib.tq_unpack_tq1(_ptr(qs), N, K, ldq, _ptr(T)), "tq_unpack_tq1")
    return T


# ------------------------------------------------------------------ device

_DTYPES = {"f16": "float16", "f32": "float32", "u8": "uint8", "i32": "int32"}


def _need(t, name, dtype, shape=None, where=""):
    """Check one device-tensor argument before its pointer reaches the C ABI,
    which receives bare pointers and cannot check sizes itself: a buffer that
    is too small would be read or written past its end.  Order: type and dtype
    (TQ_ERR_VALUE), rank, shape and contiguity (TQ_ERR_SHAPE), then device
    (TQ_ERR_DEVICE), so that every check but the last also runs without a GPU."""
    import torch
    if not torch.is_tensor(t):
        raise TQError(TQ_ERR_VALUE, f"{where}: {name} must be a torch tensor")
    if t.dtype != getattr(torch, _DTYPES[dtype]):
        raise TQError(TQ_ERR_VALUE, f"{where}: {name} must be {_DTYPES[dtype]}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise TQError(TQ_ERR_SHAPE, f"{where}: {name} has shape {tuple(t.shape)}, "
                                    f"expected {tuple(shape)}")
    if not t.is_contiguous():
        raise TQError(TQ_ERR_SHAPE, f"{where}: {name} must be contiguous (row-major)")
    return t


def _on_gpu(where, *named):
    """Every (name, tensor) on a GPU, all on the first one's device; run after
    the dtype and shape checks of every argument."""
    first = named[0][1]
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise TQError(TQ_ERR_DEVICE, f"{where}: {name} is on {t.device}, not on a GPU")
        if t.device != first.device:
            raise TQError(TQ_ERR_DEVICE, f"{where}: {name} is on {t.device}, "
                                         f"{named[0][0]} on {first.device}")


def _rank2(t, name, where):
    import torch
    if not torch.is_tensor(t) or t.dim() != 2:
        raise TQError(TQ_ERR_SHAPE, f"{where}: {name} must be a 2-D tensor")
    return t.shape


def _stream(stream, device=None):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _out(Y, M, N, where, operands, name="Y"):
    """The output: Y checked as fp16 [M][N] when given, then every operand's
    device (``operands`` as (name, tensor) pairs); a new tensor on the first
    operand's device when Y is None (allocated only after every check)."""
    import torch
    if Y is not None:
        _need(Y, name, "f16", (M, N), where)
    _on_gpu(where, *operands, (name, Y))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=operands[0][1].device)
    return Y


def _device_of(t):
    """Context that makes t's GPU the current HIP device for the C call."""
    import torch
    return torch.cuda.device(t.device)


def _gemm_operands(X, qs, scales, where, ldq_from_qs=False):
    """(M, N, K, ldq) of a product after checking X [M][K] fp16, qs [N][K/4]
    (TQ2) or [N][ldq] (TQ1) uint8 and scales [N][K/256] fp16."""
    M, K = _rank2(X, "X", where)
    N, qcols = _rank2(qs, "qs", where)
    _need(X, "X", "f16", None, where)
    _need(qs, "qs", "u8", (N, qcols if ldq_from_qs else K // 4), where)
    if not ldq_from_qs and qcols * 4 != K:
        raise TQError(TQ_ERR_SHAPE, f"{where}: qs has {qcols} bytes per row, expected K/4 = {K // 4}")
    _need(scales, "scales", "f16", (N, K // 256), where)
    return M, N, K, qcols


def tq_gemm_tq2_ex(X, qs, scales, path: int, Y=None, stream=None):
    """Y[M][N] = X[M][K] (s . T)^T for TQ2 weights qs [N][K/4]; tensors on the GPU."""
    where = "tq_gemm_tq2"
    M, N, K, _ = _gemm_operands(X, qs, scales, where)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq2_ex(_ptr(X), _ptr(qs), _ptr(scales), _ptr(Y), M, N, K, path,
                                  _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq1_ex(X, qs, scales, path: int, Y=None, stream=None):
    """Same as tq_gemm_tq2_ex for TQ1 weights qs [N][ldq] (ldq = qs.shape[1])."""
    where = "tq_gemm_tq1"
    M, N, K, ldq = _gemm_operands(X, qs, scales, where, ldq_from_qs=True)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq1_ex(_ptr(X), _ptr(qs), ldq, _ptr(scales), _ptr(Y), M, N, K, path,
                                  _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq2_tiled(X, qs, scales, mt: int, ng: int, kg: int, Y=None, stream=None):
    """tq_gemm_tq2 on the tiled kernel with an explicit (mt, ng, kg) tile."""
    where = "tq_gemm_tq2_tiled"
    M, N, K, _ = _gemm_operands(X, qs, scales, where)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq2_tiled(_ptr(X), _ptr(qs), _ptr(scales), _ptr(Y), M, N, K, mt, ng,
                                     kg, _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq2_swiglu(X, qs_gate, scales_gate, qs_up, scales_up, Y=None, stream=None):
    """silu(X G^T) * (X U^T) for TQ2 gate / up matrices, M <= 16, one launch."""
    where = "tq_gemm_tq2_swiglu"
    M, N, K, _ = _gemm_operands(X, qs_gate, scales_gate, where)
    _need(qs_up, "qs_up", "u8", tuple(qs_gate.shape), where)
    _need(scales_up, "scales_up", "f16", tuple(scales_gate.shape), where)
    Y = _out(Y, M, N, where, (("X", X), ("qs_gate", qs_gate), ("scales_gate", scales_gate),
                              ("qs_up", qs_up), ("scales_up", scales_up)))
    with _device_of(X):
        _check(lib.tq_gemm_tq2_swiglu(_ptr(X), _ptr(qs_gate), _ptr(scales_gate), _ptr(qs_up),
                                      _ptr(scales_up), _ptr(Y), M, N, K,
                                      _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq2_bwd_x(dY, qs, scales, dX=None, stream=None):
    """dX = dY (s . T): the input gradient of tq_gemm_tq2 (N % 8 == 0)."""
    where = "tq_gemm_tq2_bwd_x"
    M, N = _rank2(dY, "dY", where)
    _, qcols = _rank2(qs, "qs", where)
    K = qcols * 4
    _need(dY, "dY", "f16", None, where)
    _need(qs, "qs", "u8", (N, qcols), where)
    _need(scales, "scales", "f16", (N, K // 256), where)
    dX = _out(dX, M, K, where, (("dY", dY), ("qs", qs), ("scales", scales)), name="dX")
    with _device_of(dY):
        _check(lib.tq_gemm_tq2_bwd_x(_ptr(dY), _ptr(qs), _ptr(scales), _ptr(dX), M, N, K,
                                     _stream(stream, dY.device)), where)
    return dX


def tq_ste_grad_w(dY, X, dW=None, accumulate: bool = False, stream=None):
    """Latent-weight gradient under the straight-through estimator: dW [N][K]
    (float32) = dY^T X, or dW + dY^T X with accumulate (dW then required);
    dY fp16 [M][N], X fp16 [M][K]."""
    import torch
    where = "tq_ste_grad_w"
    M, N = _rank2(dY, "dY", where)
    M2, K = _rank2(X, "X", where)
    if M2 != M:
        raise TQError(TQ_ERR_SHAPE, f"{where}: dY has {M} rows, X {M2}")
    _need(dY, "dY", "f16", None, where)
    _need(X, "X", "f16", None, where)
    if dW is not None:
        _need(dW, "dW", "f32", (N, K), where)
    elif accumulate:
        raise TQError(TQ_ERR_NULL, f"{where}: accumulate needs dW")
    _on_gpu(where, ("dY", dY), ("X", X), ("dW", dW))
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    with _device_of(dY):
        _check(lib.tq_ste_grad_w(_ptr(dY), _ptr(X), _ptr(dW), M, N, K, int(bool(accumulate)),
                                 _stream(stream, dY.device)), where)
    return dW


def tq_tq1_transcode_min_m(N: int, K: int) -> int:
    """Activation rows from which tq_gemm_tq1_ws transcodes an N x K matrix to TQ2."""
    r = int(lib.tq_tq1_transcode_min_m(N, K))
    _check(min(r, 0), "tq_tq1_transcode_min_m")
    return r


def tq_transcode_tq1_tq2(qs1, K: int, qs2=None, stream=None):
    """TQ2 bytes [N][K/4] (uint8, device) holding the trits of the TQ1 rows qs1 [N][ldq]."""
    import torch
    where = "tq_transcode_tq1_tq2"
    N, ldq = _rank2(qs1, "qs1", where)
    _need(qs1, "qs1", "u8", None, where)
    if qs2 is not None:
        _need(qs2, "qs2", "u8", (N, K // 4), where)
    _on_gpu(where, ("qs1", qs1), ("qs2", qs2))
    if qs2 is None:
        qs2 = torch.empty((N, K // 4), dtype=torch.uint8, device=qs1.device)
    with _device_of(qs1):
        _check(lib.tq_transcode_tq1_tq2(_ptr(qs1), ldq, N, K, _ptr(qs2),
                                        _stream(stream, qs1.device)), where)
    return qs2


def tq_gemm_tq1_ws(X, qs, scales, workspace, Y=None, stream=None):
    """tq_gemm_tq1 with a workspace (uint8 device tensor of at least N * K / 4
    bytes): from tq_tq1_transcode_min_m(N, K) rows on, the weights are
    transcoded once into it and the TQ2 kernels run."""
    where = "tq_gemm_tq1_ws"
    M, N, K, ldq = _gemm_operands(X, qs, scales, where, ldq_from_qs=True)
    nbytes = 0
    if workspace is not None:
        _need(workspace, "workspace", "u8", None, where)
        nbytes = workspace.numel()
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales), ("workspace", workspace)))
    with _device_of(X):
        _check(lib.tq_gemm_tq1_ws(_ptr(X), _ptr(qs), ldq, _ptr(scales), _ptr(Y), M, N, K,
                                  _ptr(workspace), nbytes, _stream(stream, X.device)), where)
    return Y


def tq_stream_read(src, sink, stream=None):
    """Read every byte of the contiguous device tensor src once (the practical
    read ceiling); sink is an int32 device tensor of at least one element."""
    where = "tq_stream_read"
    import torch
    if not torch.is_tensor(src):
        raise TQError(TQ_ERR_VALUE, f"{where}: src must be a torch tensor")
    if not src.is_contiguous():
        raise TQError(TQ_ERR_SHAPE, f"{where}: src must be contiguous")
    _need(sink, "sink", "i32", None, where)
    if sink.numel() < 1:
        raise TQError(TQ_ERR_SHAPE, f"{where}: sink needs at least one int32")
    _on_gpu(where, ("src", src), ("sink", sink))
    nbytes = src.numel() * src.element_size()
    with _device_of(src):
        _check(lib.tq_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream, src.device)),
               where)


def tq_gemm_tq2_tile(X, qs, scales, mt: int, nr: int, ng: int, kg: int, Y=None, stream=None):
    """tq_gemm_tq2 on the tiled kernel with an explicit (mt, nr, ng, kg) tile."""
    where = "tq_gemm_tq2_tile"
    M, N, K, _ = _gemm_operands(X, qs, scales, where)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq2_tile(_ptr(X), _ptr(qs), _ptr(scales), _ptr(Y), M, N, K, mt, nr, ng,
                                    kg, _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq2_wide(X, qs, scales, mt: int, nt: int, ng: int, kg: int, Y=None, stream=None):
    """tq_gemm_tq2 on the wide-tile kernel with an explicit (mt, nt, ng, kg) tile."""
    where = "tq_gemm_tq2_wide"
    M, N, K, _ = _gemm_operands(X, qs, scales, where)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq2_wide(_ptr(X), _ptr(qs), _ptr(scales), _ptr(Y), M, N, K, mt, nt, ng,
                                    kg, _stream(stream, X.device)), where)
    return Y


def tq_gemm_tq1_tile(X, qs, scales, mt: int, nr: int, ng: int, kg: int, Y=None, stream=None):
    """tq_gemm_tq1 on the table-decode tiled kernel with an explicit tile."""
    where = "tq_gemm_tq1_tile"
    M, N, K, ldq = _gemm_operands(X, qs, scales, where, ldq_from_qs=True)
    Y = _out(Y, M, N, where, (("X", X), ("qs", qs), ("scales", scales)))
    with _device_of(X):
        _check(lib.tq_gemm_tq1_tile(_ptr(X), _ptr(qs), ldq, _ptr(scales), _ptr(Y), M, N, K, mt,
                                    nr, ng, kg, _stream(stream, X.device)), where)
    return Y


def tq_pack_dev(fmt: int, W, eps: float = 1e-5, ldq: int | None = None, stream=None):
    """On-device ternarize + pack of a float32 [N][K] device tensor W (fmt 2 or 1).
    Returns device tensors (qs, scales fp16, gamma fp64 [1], status int32 [1])."""
    import torch
    where = "tq_pack_tq%d_dev" % fmt
    if fmt not in (1, 2):
        raise TQError(TQ_ERR_VALUE, f"{where}: format must be 1 or 2")
    N, K = _rank2(W, "W", where)
    _need(W, "W", "f32", None, where)
    _on_gpu(where, ("W", W))
    dev = W.device
    if fmt == 2:
        qs = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    else:
        ldq = tq_tq1_ldq(K) if ldq is None else ldq
        qs = torch.empty((N, max(ldq, 0)), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 256), dtype=torch.float16, device=dev)
    gamma = torch.empty(1, dtype=torch.float64, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    wsb = lib.tq_pack_dev_workspace_bytes(N, K)
    if wsb < 0:
        raise TQError(TQ_ERR_SHAPE, "tq_pack_dev_workspace_bytes")
    ws = torch.empty(int(wsb), dtype=torch.uint8, device=dev)
    with _device_of(W):
        sp = _stream(stream, dev)
        if fmt == 2:
            st = lib.tq_pack_tq2_dev(_ptr(W), N, K, float(eps), _ptr(qs), _ptr(scales),
                                     _ptr(gamma), _ptr(status), _ptr(ws), wsb, sp)
        else:
            st = lib.tq_pack_tq1_dev(_ptr(W), N, K, float(eps), ldq, _ptr(qs), _ptr(scales),
                                     _ptr(gamma), _ptr(status), _ptr(ws), wsb, sp)
    _check(st, where)
    return qs, scales, gamma, status


def tq_pack_tq2_dev_noalloc(W, qs, scales, gamma, status, eps: float = 1e-5, stream=None):
    """tq_pack_tq2_dev into caller-owned outputs with the library's fixed
    per-device workspace (no device allocation by this call): W float32
    [N][K], qs uint8 [N][K/4], scales fp16 [N][K/256], gamma float64 [1],
    status int32 [1], all on one GPU."""
    import torch
    where = "tq_pack_tq2_dev_noalloc"
    N, K = _rank2(W, "W", where)
    _need(W, "W", "f32", None, where)
    _need(qs, "qs", "u8", (N, K // 4), where)
    _need(scales, "scales", "f16", (N, K // 256), where)
    if not (torch.is_tensor(gamma) and gamma.dtype == torch.float64 and gamma.numel() >= 1):
        raise TQError(TQ_ERR_VALUE, f"{where}: gamma must be a float64 tensor of >= 1 element")
    if not (torch.is_tensor(status) and status.dtype == torch.int32 and status.numel() >= 1):
        raise TQError(TQ_ERR_VALUE, f"{where}: status must be an int32 tensor of >= 1 element")
    _on_gpu(where, ("W", W), ("qs", qs), ("scales", scales), ("gamma", gamma), ("status", status))
    with _device_of(W):
        _check(lib.tq_pack_tq2_dev_noalloc(_ptr(W), N, K, float(eps), _ptr(qs), _ptr(scales),
                                           _ptr(gamma), _ptr(status), _stream(stream, W.device)),
               where)


def tq_gemm_tq2(X, qs, scales, Y=None, stream=None):
    return tq_gemm_tq2_ex(X, qs, scales, TQ_PATH_AUTO, Y, stream)


def tq_gemm_tq1(X, qs, scales, Y=None, stream=None):
    return tq_gemm_tq1_ex(X, qs, scales, TQ_PATH_AUTO, Y, stream)


def tq_kernel_name(fmt: int, M: int, N: int, K: int, path: int = TQ_PATH_AUTO) -> str:
    """Kernel that the product with this format (2 or 1), shape and path runs."""
    buf = C.create_string_buffer(128)
    _check(lib.tq_kernel_name(fmt, M, N, K, path, buf, 128), "tq_kernel_name")
    return buf.value.decode()


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw arguments and return its status (for tests)."""
    return getattr(lib, name)(*args)
