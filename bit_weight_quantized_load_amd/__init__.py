"""Weight-quantized decode linear (W4A8 / W8A16 GEMV) for AMD MI355X.

A thin ctypes binding over the C ABI in ``include/qwgemv.h`` (``libqwgemv.so``,
hand-written HIP for gfx950).  The functions below only marshal arguments: they
take torch tensors for device memory and the current stream, allocate outputs with
``torch.empty`` and call the library.  Every arithmetic step runs in the HIP
kernels; there is no fallback, and importing the compute functions without the
built library raises.

W4A8 follows "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s"
(sections 正确方向 and 当前实现方式; the group-wise variant is the scale granularity its
section 后续优化方向 lists as future work); W8A16 follows the ChatGLM2-6B W8A16 write-up
(TPU-MLIR, sections 2-4).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwgemv.so")

QW_OK = 0
QW_ERR_NULL = 1
QW_ERR_SHAPE = 2
QW_ERR_ALIGN = 3
QW_ERR_WORKSPACE = 4
QW_ERR_NONFINITE = 5
QW_ERR_HIP = 6
QW_ERR_TILING = 7

# name -> (restype, argtypes) for every entry point of include/qwgemv.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_I = ctypes.c_int
SIGNATURES = {
    "qw_w4_packed_bytes": (_SZ, [_I64, _I64]),
    "qw_w8_packed_bytes": (_SZ, [_I64, _I64]),
    "qw_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "qw_workspace_clear": (_I, [_P, _SZ, _P]),
    "quantize_pack_w4": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "quantize_pack_w8": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "quant_act_i8": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "gemv_w4a8": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "gemv_w8a16": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "gemv_w4a8_noalloc": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "qw_w4_codes": (_I, [_P, _I64, _I64, _P, _P]),
    "qw_w8_codes": (_I, [_P, _I64, _I64, _P, _P]),
    "qw_gemv_w4a8_debug": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "qw_gemv_w4a8_tiled": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _I, _I, _I, _P]),
    "qw_gemv_w8a16_tiled": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _I, _I, _I, _P]),
    "qw_gemm_w4a8_mfma": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _I, _I, _I, _P]),
    "qw_gemv_w4a8_long_k": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _I, _I, _P]),
    "qw_gemm_w8a16_mfma": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _I, _I, _P]),
    "qw_gemm_w8a16_tile": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "qw_gemm_w4a8_tile": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _I, _P]),
    "qw_tile_variant": (_I, [_I, _I64, _I64]),
    "qw_w4g_scale_bytes": (_SZ, [_I64, _I64, _I64]),
    "quantize_pack_w4g": (_I, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "qw_w4g_scales": (_I, [_P, _I64, _I64, _I64, _P, _P]),
    "gemv_w4a8g": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "qw_gemv_w4a8g_tiled": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _I, _I, _I, _P]),
    "qw_gemv_f16": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "qw_gemv_w4f32": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "index_softmax": (_I, [_P, _I64, _I64, ctypes.c_int32, _I, ctypes.c_double, _P, _P]),
    "qw_index_cint": (ctypes.c_int32, [ctypes.c_double, _I64, ctypes.c_double, ctypes.c_double]),
    "qw_index_magic": (_I, [ctypes.c_int32, _I, _P, _P]),
    "qw_status_str": (ctypes.c_char_p, [_I]),
    "qw_last_hip_error": (_I, []),
    "qw_device_status": (_I, [_P, _I]),
    "qw_stream_read": (_I, [_P, _SZ, _P, _I, _I, _I, _P]),
}


class QWError(RuntimeError):
    def __init__(self, fn: str, status: int, lib=None):
        msg = lib.qw_status_str(status).decode() if lib is not None else "status %d" % status
        if status == QW_ERR_HIP and lib is not None:
            msg += " (hipError %d)" % lib.qw_last_hip_error()
        super().__init__("%s: %s" % (fn, msg))
        self.status = status


_lib = None


def lib():
    """The loaded libqwgemv.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libqwgemv.so is not built (%s); run __graft_entry__.build() or "
                "python -m bit_weight_quantized_load_amd._build" % LIB_PATH)
        # torch ships its own HIP runtime (same soname, libamdhip64.so.7).  Loading
        # torch first makes the library bind to that one runtime instead of bringing
        # a second copy of the runtime into the process.
        import torch  # noqa: F401

        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _call(name, *args):
    L = lib()
    st = getattr(L, name)(*args)
    if st != QW_OK:
        raise QWError(name, st, L)


# ----------------------------------------------------------------- torch side --

def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, shape, name):
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_bytes(op: str, M: int, N: int, K: int) -> int:
    return int(lib().qw_workspace_bytes(0 if op == "w4a8" else 1, M, N, K))


def make_workspace(op: str, M: int, N: int, K: int, device="cuda", stream=None):
    """A zero-filled workspace for gemv_<op> at shape (M, N, K), or None if none is needed."""
    nbytes = workspace_bytes(op, M, N, K)
    if nbytes == 0:
        return None
    torch = _torch()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _call("qw_workspace_clear", _ptr(ws), nbytes, _stream(stream))
    return ws


def w4_packed_bytes(N: int, K: int) -> int:
    return int(lib().qw_w4_packed_bytes(N, K))


def w8_packed_bytes(N: int, K: int) -> int:
    return int(lib().qw_w8_packed_bytes(N, K))


def quantize_pack_w4(W, stream=None):
    """W fp32 [N][K] -> (Wq uint8 [w4_packed_bytes(N, K)] in the tile layout, w_scale fp32 [N]).
    Load time; synchronises."""
    torch = _torch()
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    Wq = torch.empty((w4_packed_bytes(N, K),), dtype=torch.uint8, device=W.device)
    s = torch.empty((N,), dtype=torch.float32, device=W.device)
    _call("quantize_pack_w4", _ptr(W), N, K, _ptr(Wq), _ptr(s), _stream(stream))
    return Wq, s


def quantize_pack_w8(W, stream=None):
    """W fp32 [N][K] -> (Wq uint8 [w8_packed_bytes(N, K)] in the tile layout, w_scale fp16 [N]).
    Load time; synchronises."""
    torch = _torch()
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    Wq = torch.empty((w8_packed_bytes(N, K),), dtype=torch.uint8, device=W.device)
    s = torch.empty((N,), dtype=torch.float16, device=W.device)
    _call("quantize_pack_w8", _ptr(W), N, K, _ptr(Wq), _ptr(s), _stream(stream))
    return Wq, s


def quant_act_i8(X, stream=None):
    """X fp32 [M][K] -> (Xq int8 [M][K], a_scale fp32 [M])."""
    torch = _torch()
    M, K = X.shape
    _need(X, torch.float32, (M, K), "X")
    Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    a = torch.empty((M,), dtype=torch.float32, device=X.device)
    _call("quant_act_i8", _ptr(X), M, K, _ptr(Xq), _ptr(a), _stream(stream))
    return Xq, a


def _ws_args(ws):
    if ws is None:
        return ctypes.c_void_p(0), 0
    return _ptr(ws), ws.numel() * ws.element_size()


def gemv_w4a8(X, Wq, w_scale, workspace=None, out=None, stream=None):
    """Y fp32 [M][N] = W4A8 linear of X fp32 [M][K] (activation quantization fused)."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    wp, wn = _ws_args(workspace)
    _call("gemv_w4a8", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), wp, wn, _stream(stream))
    return Y


def gemv_w4a8_noalloc(X, Wq, w_scale, out=None, stream=None):
    """gemv_w4a8 without a workspace: from two rows of X the library's fixed per-GPU
    scratch array (8 MiB) holds the activation codes; larger shapes raise QWError
    (QW_ERR_WORKSPACE).  Calls overlapping on one GPU race."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    _call("gemv_w4a8_noalloc", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), _stream(stream))
    return Y


def gemv_w4a8_debug(X, Wq, w_scale, workspace=None, stream=None):
    """gemv_w4a8 that also returns the int32 accumulators and the prologue's codes/scales."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    dev = X.device
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    a = torch.empty((M,), dtype=torch.float32, device=dev)
    wp, wn = _ws_args(workspace)
    _call("qw_gemv_w4a8_debug", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), _ptr(acc),
          _ptr(xq), _ptr(a), wp, wn, _stream(stream))
    return {"Y": Y, "acc": acc, "xq": xq, "a": a}


def gemv_w8a16(X16, Wq, w_scale16, workspace=None, out=None, stream=None):
    """Y fp16 [M][N] = W8A16 linear of X fp16 [M][K]."""
    torch = _torch()
    M, K = X16.shape
    N = w_scale16.shape[0]
    _need(X16, torch.float16, (M, K), "X16")
    _need(Wq, torch.uint8, (w8_packed_bytes(N, K),), "Wq")
    _need(w_scale16, torch.float16, (N,), "w_scale16")
    Y = torch.empty((M, N), dtype=torch.float16, device=X16.device) if out is None else out
    _need(Y, torch.float16, (M, N), "out")
    wp, wn = _ws_args(workspace)
    _call("gemv_w8a16", _ptr(X16), _ptr(Wq), _ptr(w_scale16), M, N, K, _ptr(Y), wp, wn,
          _stream(stream))
    return Y


def w4g_scale_bytes(N: int, K: int, group: int) -> int:
    return int(lib().qw_w4g_scale_bytes(N, K, group))


def quantize_pack_w4g(W, group, stream=None):
    """W fp32 [N][K] -> (Wq uint8 [w4_packed_bytes(N, K)], group scales fp32 in the device
    layout [w4g_scale_bytes(N, K, group) / 4]), one scale per output row and group of
    `group` consecutive k.  Load time; synchronises."""
    torch = _torch()
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    nb = w4g_scale_bytes(N, K, group)
    if nb == 0:
        raise QWError("quantize_pack_w4g", QW_ERR_SHAPE, lib())
    Wq = torch.empty((w4_packed_bytes(N, K),), dtype=torch.uint8, device=W.device)
    s = torch.empty((nb // 4,), dtype=torch.float32, device=W.device)
    _call("quantize_pack_w4g", _ptr(W), N, K, group, _ptr(Wq), _ptr(s), _stream(stream))
    return Wq, s


def w4g_scales(w_scale, N, K, group, stream=None):
    """Group scales in the device layout -> fp32 [N][K / group]."""
    torch = _torch()
    out = torch.empty((N, K // group), dtype=torch.float32, device=w_scale.device)
    _call("qw_w4g_scales", _ptr(w_scale), N, K, group, _ptr(out), _stream(stream))
    return out


def gemv_w4a8g(X, Wq, w_scale, N, group, out=None, stream=None):
    """Y fp32 [1][N] = group-wise W4A8 linear of X fp32 [1][K] (M == 1)."""
    torch = _torch()
    M, K = X.shape
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (w4g_scale_bytes(N, K, group) // 4,), "w_scale")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    _call("gemv_w4a8g", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, group, _ptr(Y), None, 0,
          _stream(stream))
    return Y


def gemv_w4a8g_tiled(X, Wq, w_scale, N, group, u, nw, nwaves, splitk, out=None, stream=None):
    """gemv_w4a8g with an explicit launch shape (see include/qwgemv.h)."""
    torch = _torch()
    M, K = X.shape
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _call("qw_gemv_w4a8g_tiled", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, group, _ptr(Y),
          u, nw, nwaves, splitk, _stream(stream))
    return Y


def gemv_w4a8_tiled(X, Wq, w_scale, u, nw, nwaves, splitk=1, out=None, stream=None):
    """gemv_w4a8 with an explicit launch shape (see include/qwgemv.h)."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _call("qw_gemv_w4a8_tiled", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y),
          u, nw, nwaves, splitk, _stream(stream))
    return Y


def gemv_w8a16_tiled(X16, Wq, w_scale16, u, nw, nwaves, splitk=1, out=None, stream=None):
    """gemv_w8a16 with an explicit launch shape (see include/qwgemv.h)."""
    torch = _torch()
    M, K = X16.shape
    N = w_scale16.shape[0]
    _need(X16, torch.float16, (M, K), "X16")
    _need(Wq, torch.uint8, (w8_packed_bytes(N, K),), "Wq")
    Y = torch.empty((M, N), dtype=torch.float16, device=X16.device) if out is None else out
    _call("qw_gemv_w8a16_tiled", _ptr(X16), _ptr(Wq), _ptr(w_scale16), M, N, K, _ptr(Y),
          u, nw, nwaves, splitk, _stream(stream))
    return Y


def gemm_w4a8_mfma(X, Wq, w_scale, nw=4, mb=1, nbw=1, workspace=None, out=None, stream=None):
    """The W4A8 matrix-core kernel at any M with an explicit launch shape (nw waves per
    workgroup, mb blocks of 16 rows of X per workgroup, nbw blocks of 16 output rows
    per wave).  Needs a workspace of qw_workspace_bytes(2, M, N, K) bytes."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if workspace is None:
        workspace = torch.empty((lib().qw_workspace_bytes(2, M, N, K),), dtype=torch.uint8,
                                device=X.device)
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    wp, wn = _ws_args(workspace)
    _call("qw_gemm_w4a8_mfma", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), wp, wn,
          nw, mb, nbw, _stream(stream))
    return Y


def gemv_w4a8_long_k(X, Wq, w_scale, waves, workgroups, workspace=None, out=None, stream=None):
    """The balanced long-K W4A8 kernel at any M with an explicit launch shape (`waves`
    k-slices per workgroup, `workgroups` workgroups).  Needs a workspace of
    qw_workspace_bytes(2, M, N, K) bytes."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if workspace is None:
        workspace = torch.empty((lib().qw_workspace_bytes(2, M, N, K),), dtype=torch.uint8,
                                device=X.device)
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    wp, wn = _ws_args(workspace)
    _call("qw_gemv_w4a8_long_k", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), wp, wn,
          waves, workgroups, _stream(stream))
    return Y


def gemm_w8a16_mfma(X16, Wq, w_scale16, nw=4, mb=1, nbw=1, out=None, stream=None):
    """The W8A16 matrix-core kernel at any M with an explicit launch shape."""
    torch = _torch()
    M, K = X16.shape
    N = w_scale16.shape[0]
    _need(X16, torch.float16, (M, K), "X16")
    _need(Wq, torch.uint8, (w8_packed_bytes(N, K),), "Wq")
    _need(w_scale16, torch.float16, (N,), "w_scale16")
    Y = torch.empty((M, N), dtype=torch.float16, device=X16.device) if out is None else out
    _need(Y, torch.float16, (M, N), "out")
    _call("qw_gemm_w8a16_mfma", _ptr(X16), _ptr(Wq), _ptr(w_scale16), M, N, K, _ptr(Y),
          nw, mb, nbw, _stream(stream))
    return Y


def gemm_w8a16_tile(X16, Wq, w_scale16, variant=0, out=None, stream=None):
    """The tiled f16 matrix-core W8A16 GEMM at launch variant 0 to 8 (output tiles of
    256 x 256, 256 x 128, 128 x 128, 128 x 128 in two k-groups, 128 x 64, 128 x 64 in
    two k-groups, 64 x 64, 128 x 64 in two k-groups with deeper stages, and 128 x 32
    with deeper stages: rows of W by rows of X)."""
    torch = _torch()
    M, K = X16.shape
    N = w_scale16.shape[0]
    _need(X16, torch.float16, (M, K), "X16")
    _need(Wq, torch.uint8, (w8_packed_bytes(N, K),), "Wq")
    _need(w_scale16, torch.float16, (N,), "w_scale16")
    Y = torch.empty((M, N), dtype=torch.float16, device=X16.device) if out is None else out
    _need(Y, torch.float16, (M, N), "out")
    _call("qw_gemm_w8a16_tile", _ptr(X16), _ptr(Wq), _ptr(w_scale16), M, N, K, _ptr(Y), int(variant),
          _stream(stream))
    return Y


def gemm_w4a8_tile(X, Wq, w_scale, variant=0, workspace=None, out=None, stream=None):
    """The tiled int8 matrix-core W4A8 GEMM at a launch variant (see gemm_w8a16_tile);
    the workspace (op 2 size) is allocated when not given."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if workspace is None:
        workspace = torch.empty(int(lib().qw_workspace_bytes(2, M, N, K)), dtype=torch.uint8,
                                device=X.device)
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    wp, wn = _ws_args(workspace)
    _call("qw_gemm_w4a8_tile", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), wp, wn, int(variant),
          _stream(stream))
    return Y


def gemv_f16(X16, W16, rows_per_wave=0, out=None, stream=None):
    """The FP16 baseline GEMV (an ablation): Y f16 [1][N] of X16 f16 [1][K] and row-major
    W16 f16 [N][K]."""
    torch = _torch()
    M, K = X16.shape
    N = W16.shape[0]
    _need(X16, torch.float16, (M, K), "X16")
    _need(W16, torch.float16, (N, K), "W16")
    Y = torch.empty((M, N), dtype=torch.float16, device=X16.device) if out is None else out
    _need(Y, torch.float16, (M, N), "out")
    _call("qw_gemv_f16", _ptr(X16), _ptr(W16), M, N, K, _ptr(Y), rows_per_wave, _stream(stream))
    return Y


def gemv_w4f32(X, Wq, w_scale, rows_per_wave=0, out=None, stream=None):
    """Weight-only INT4 with float activations (an ablation): Y fp32 [1][N]."""
    torch = _torch()
    M, K = X.shape
    N = w_scale.shape[0]
    _need(X, torch.float32, (M, K), "X")
    _need(Wq, torch.uint8, (w4_packed_bytes(N, K),), "Wq")
    _need(w_scale, torch.float32, (N,), "w_scale")
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    _need(Y, torch.float32, (M, N), "out")
    _call("qw_gemv_w4f32", _ptr(X), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y), rows_per_wave,
          _stream(stream))
    return Y


def index_cint(c, d, s_q, s_k) -> int:
    """IndexSoftmax clipping threshold round(c * sqrt(d) / (s_Q * s_K)) (-1 if invalid)."""
    return int(lib().qw_index_cint(float(c), int(d), float(s_q), float(s_k)))


def index_softmax(A, c_int, b=5, c=6.6, out=None, stream=None):
    """IndexSoftmax of int32 logits A [rows][L] -> UINT8 probabilities [rows][L]."""
    torch = _torch()
    rows, L = A.shape
    _need(A, torch.int32, (rows, L), "A")
    P = torch.empty((rows, L), dtype=torch.uint8, device=A.device) if out is None else out
    _need(P, torch.uint8, (rows, L), "out")
    _call("index_softmax", _ptr(A), rows, L, int(c_int), int(b), float(c), _ptr(P), _stream(stream))
    return P


def w4_codes(Wq, N, K, stream=None):
    torch = _torch()
    codes = torch.empty((N, K), dtype=torch.int8, device=Wq.device)
    _call("qw_w4_codes", _ptr(Wq), N, K, _ptr(codes), _stream(stream))
    return codes


def w8_codes(Wq, N, K, stream=None):
    torch = _torch()
    codes = torch.empty((N, K), dtype=torch.int8, device=Wq.device)
    _call("qw_w8_codes", _ptr(Wq), N, K, _ptr(codes), _stream(stream))
    return codes


def device_status(clear: bool = True) -> int:
    """The library's device status word on the current device (QW_STATUS_* bits; 0 when
    every fused activation quantization since the last clear ran as designed)."""
    out = ctypes.c_uint32(0)
    _call("qw_device_status", ctypes.byref(out), 1 if clear else 0)
    return int(out.value)


QW_STATUS_PRODUCER_WAIT = 1


def stream_read(src, sink, waves=0, blocks=0, loads_in_flight=0, stream=None):
    """Bandwidth reference: the kernel reads every byte of the contiguous device tensor
    ``src`` once and writes one XOR word per workgroup into ``sink`` (uint32 or int32,
    at least ``blocks`` words; ``blocks`` 0 = one workgroup per compute unit)."""
    torch = _torch()
    if not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous device tensor")
    if sink.device.type != "cuda" or sink.dtype not in (torch.int32, torch.uint32):
        raise ValueError("sink must be a 32-bit device tensor")
    need = blocks if blocks else torch.cuda.get_device_properties(src.device).multi_processor_count
    if sink.numel() < need or not sink.is_contiguous():
        raise ValueError("sink needs %d contiguous words" % need)
    _call("qw_stream_read", _ptr(src), src.numel() * src.element_size(), _ptr(sink), int(waves),
          int(blocks), int(loads_in_flight), _stream(stream))
    return sink
