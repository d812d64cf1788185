"""CPU oracle for the weight-quantized decode linear (W4A8 and W8A16).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It wraps the plain
C99 implementation in ``qw_oracle.c`` (compiled with gcc, never with hipcc) and
shares no code with the HIP library.

Every function takes and returns numpy arrays on the host.  What each one computes,
and which passage of the pages it follows, is stated in ``qw_oracle.c``:

* ``quant_w4`` / ``pack_w4`` / ``unpack_w4`` -- row-wise INT4 weights, one scale
  per output row ("Jetson Orin AGX 上的 INT4 量化推理实践", section 当前实现方式).
* ``quant_act_i8`` -- dynamic per-vector INT8 activation quantization (same section).
* ``gemv_w4a8`` -- int32 dot of the codes, output acc * w_scale * a_scale (sections
  正确方向 and 当前实现方式).
* ``quant_w4g`` / ``gemv_w4a8g`` -- group-wise INT4 scales (one per output row and
  group of g consecutive k), per-group int32 dots summed in fp32 (the same page,
  section 后续优化方向, which lists group-wise scales as future work).
* ``quant_w8`` / ``gemv_w8a16_ref64`` -- per-channel INT8 weights with an f16
  scale, dequantize-then-matmul in fp64 (ChatGLM2-6B W8A16 write-up, sections 2-4).
* ``gemv_f16_ref64`` / ``gemv_w4f32`` -- the two ablations the INT4 page times beside
  W4A8 (section 速度结果): an FP16 GEMV (fp64 reference) and weight-only INT4 with
  float activations, unpacked to float and multiplied-added in fp32 (sections 最初的问题
  and 问题原因).
* ``index_lut`` / ``index_cint`` / ``index_softmax`` / ``int_attention`` -- IndexSoftmax, the
  integer softmax of the IntAttention summary (sections 基准/方法设计 and 方法细节).
* ``f16_from_f32`` / ``f32_from_f16`` -- IEEE binary16 conversions written from the
  format's definition.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qw_oracle.c")
_LIB = os.path.join(_HERE, "libqwo.so")

GCC_FLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile qw_oracle.c with gcc into libqwo.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        sig = {
            "qwo_quant_w4": [P, I64, I64, P, P],
            "qwo_pack_w4": [P, I64, I64, P],
            "qwo_unpack_w4": [P, I64, I64, P],
            "qwo_quant_act_i8": [P, I64, I64, P, P],
            "qwo_gemv_w4a8": [P, P, P, I64, I64, I64, P, P, P, P, ctypes.c_int],
            "qwo_quant_w4g": [P, I64, I64, I64, P, P],
            "qwo_gemv_w4a8g": [P, P, P, I64, I64, I64, I64, P, P, P, P, ctypes.c_int],
            "qwo_gemv_f16_ref64": [P, P, I64, I64, I64, P, ctypes.c_int],
            "qwo_gemv_w4f32": [P, P, P, I64, I64, I64, P, P, ctypes.c_int],
            "qwo_index_lut": [ctypes.c_int, ctypes.c_double, P],
            "qwo_index_softmax": [P, I64, I64, ctypes.c_int32, ctypes.c_int, P, P, P, ctypes.c_int],
            "qwo_int_attention": [P, P, P, I64, I64, I64, ctypes.c_int, ctypes.c_double, P, P, P, P],
            "qwo_quant_w8": [P, I64, I64, P, P],
            "qwo_gemv_w8a16_ref64": [P, P, P, I64, I64, I64, P, ctypes.c_int],
            "qwo_f16_from_f32_n": [P, I64, P],
            "qwo_f32_from_f16_n": [P, I64, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int if not name.endswith("_n") else None
        lib.qwo_num_threads.restype = ctypes.c_int
        lib.qwo_index_cint.restype = ctypes.c_int32
        lib.qwo_index_cint.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st):
    if st == 1:
        raise OracleError("bad argument")
    if st == 2:
        raise OracleError("non-finite input")
    if st != 0:
        raise OracleError("status %d" % st)


def num_threads() -> int:
    return _load().qwo_num_threads()


def quant_w4(W):
    """W fp32 [N][K] -> (codes int8 [N][K] in -7..7, scale fp32 [N])."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N,), np.float32)
    _check(_load().qwo_quant_w4(_p(W), N, K, _p(q), _p(s)))
    return q, s


def pack_w4(q):
    """codes int8 [N][K] -> canonical packed bytes uint8 [N][K/2]."""
    q = _c(q, np.int8)
    N, K = q.shape
    out = np.empty((N, K // 2), np.uint8)
    _check(_load().qwo_pack_w4(_p(q), N, K, _p(out)))
    return out


def unpack_w4(packed, K):
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    _check(_load().qwo_unpack_w4(_p(packed), N, K, _p(q)))
    return q


def quant_act_i8(X):
    """X fp32 [M][K] -> (codes int8 [M][K] in -127..127, scale fp32 [M])."""
    X = _c(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    xq = np.empty((M, K), np.int8)
    a = np.empty((M,), np.float32)
    _check(_load().qwo_quant_act_i8(_p(X), M, K, _p(xq), _p(a)))
    return xq, a


def gemv_w4a8(X, q, s, nthreads: int = 1):
    """W4A8 linear.  X fp32 [M][K], q int8 codes [N][K], s fp32 [N].

    Returns dict with Y fp32 [M][N], acc int32 [M][N], xq int8 [M][K], a fp32 [M].
    """
    X = _c(X, np.float32)
    if X.ndim == 1:
        X = X[None, :]
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    M, K = X.shape
    N = q.shape[0]
    assert q.shape == (N, K) and s.shape == (N,)
    Y = np.empty((M, N), np.float32)
    acc = np.empty((M, N), np.int32)
    xq = np.empty((M, K), np.int8)
    a = np.empty((M,), np.float32)
    _check(_load().qwo_gemv_w4a8(_p(X), _p(q), _p(s), M, N, K, _p(Y), _p(acc), _p(xq), _p(a),
                                 int(nthreads)))
    return {"Y": Y, "acc": acc, "xq": xq, "a": a}


def quant_w4g(W, g):
    """W fp32 [N][K] -> (codes int8 [N][K] in -7..7, scales fp32 [N][K/g]), one scale per
    output row and group of g consecutive k."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // g if g > 0 else 0), np.float32)
    _check(_load().qwo_quant_w4g(_p(W), N, K, int(g), _p(q), _p(s)))
    return q, s


def gemv_w4a8g(X, q, s, g, nthreads=1):
    """Group-wise W4A8 linear; returns dict Y fp32 [M][N], accg int32 [M][N][K/g] (the
    per-group dots), xq int8 [M][K], a fp32 [M]."""
    X = _c(X, np.float32)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    M, K = X.shape
    N = q.shape[0]
    G = K // g
    assert q.shape == (N, K) and s.shape == (N, G)
    Y = np.empty((M, N), np.float32)
    accg = np.empty((M, N, G), np.int32)
    xq = np.empty((M, K), np.int8)
    a = np.empty((M,), np.float32)
    _check(_load().qwo_gemv_w4a8g(_p(X), _p(q), _p(s), M, N, K, int(g), _p(Y), _p(accg), _p(xq),
                                  _p(a), int(nthreads)))
    return {"Y": Y, "accg": accg, "xq": xq, "a": a}


def w4a8g_ref64(accg, s, a):
    """fp64 value of the group-wise output from exact per-group dots: sum over groups of
    acc * s, times a (each product is exact in fp64), and the fp32 error bound
    (G + 2) * 2^-24 * sum |acc * s| * |a| that any summation order of the fp32 terms
    meets.  Returns (y64 [M][N], bound [M][N])."""
    t = accg.astype(np.float64) * s.astype(np.float64)[None, :, :]
    a64 = a.astype(np.float64)[:, None]
    G = accg.shape[2]
    y64 = t.sum(axis=2) * a64
    bound = (G + 2) * 2.0 ** -24 * np.abs(t).sum(axis=2) * np.abs(a64)
    return y64, bound


def gemv_f16_ref64(X16, W16, nthreads=1):
    """fp64 value of the FP16 GEMV: X16 f16 [M][K], W16 f16 [N][K] -> float64 [M][N]."""
    X16 = _c(X16, np.float16).view(np.uint16)
    W16 = _c(W16, np.float16).view(np.uint16)
    M, K = X16.shape
    N = W16.shape[0]
    Y64 = np.empty((M, N), np.float64)
    _check(_load().qwo_gemv_f16_ref64(_p(X16), _p(W16), M, N, K, _p(Y64), int(nthreads)))
    return Y64


def gemv_w4f32(X, q, s, nthreads=1):
    """Weight-only INT4, float activations: (Y fp32 [M][N], Y64 float64 [M][N])."""
    X = _c(X, np.float32)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    M, K = X.shape
    N = q.shape[0]
    Y = np.empty((M, N), np.float32)
    Y64 = np.empty((M, N), np.float64)
    _check(_load().qwo_gemv_w4f32(_p(X), _p(q), _p(s), M, N, K, _p(Y), _p(Y64), int(nthreads)))
    return Y, Y64


def w4f32_bound(X, q, s):
    """Per-element bound (K + 2) * 2^-24 * s[n] * sum_k |q x| on |Y - Y64| for any order of
    the K fp32 multiply-adds (and the final scale multiply)."""
    K = X.shape[1]
    t = np.abs(X.astype(np.float64)) @ np.abs(q.astype(np.float64)).T
    return (K + 2) * 2.0 ** -24 * t * s.astype(np.float64)[None, :]


def index_lut(b=5, c=6.6):
    """The 2^b-entry UINT8 exponent table of IndexSoftmax."""
    lut = np.empty((1 << b,), np.uint8)
    _check(_load().qwo_index_lut(int(b), float(c), _p(lut)))
    return lut


def index_cint(c, d, s_q, s_k):
    """Integer clipping threshold round(c * sqrt(d) / (s_Q * s_K))."""
    return int(_load().qwo_index_cint(float(c), int(d), float(s_q), float(s_k)))


def index_softmax(A, c_int, b=5, c=6.6, nthreads=1):
    """IndexSoftmax of int32 logits A [rows][L] -> (P uint8 [rows][L], rowSum int32 [rows])."""
    A = _c(A, np.int32)
    rows, L = A.shape
    lut = index_lut(b, c)
    P = np.empty((rows, L), np.uint8)
    rs = np.empty((rows,), np.int32)
    _check(_load().qwo_index_softmax(_p(A), rows, L, int(c_int), int(b), _p(lut), _p(P), _p(rs),
                                     int(nthreads)))
    return P, rs


def int_attention(Q, K, V, b=5, c=6.6):
    """One head of the all-integer attention: dict A int32, P uint8, O fp32, c_int."""
    Q = _c(Q, np.float32)
    K = _c(K, np.float32)
    V = _c(V, np.float32)
    Lq, d = Q.shape
    Lk = K.shape[0]
    if K.shape != (Lk, d) or V.shape != (Lk, d):
        raise ValueError("K and V must be [Lk][d] with the d of Q [Lq][d]")
    A = np.empty((Lq, Lk), np.int32)
    P = np.empty((Lq, Lk), np.uint8)
    O = np.empty((Lq, d), np.float32)
    ci = np.zeros((1,), np.int32)
    _check(_load().qwo_int_attention(_p(Q), _p(K), _p(V), Lq, Lk, d, int(b), float(c), _p(A), _p(P),
                                     _p(O), _p(ci)))
    return {"A": A, "P": P, "O": O, "c_int": int(ci[0])}


def quant_w8(W):
    """W fp32 [N][K] -> (codes int8 [N][K] in -127..127, scale f16 bits uint16 [N])."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s16 = np.empty((N,), np.uint16)
    _check(_load().qwo_quant_w8(_p(W), N, K, _p(q), _p(s16)))
    return q, s16


def gemv_w8a16_ref64(X16, q, s16, nthreads: int = 1):
    """W8A16 linear in fp64.  X16 f16 bits [M][K] (uint16 or float16), q int8 [N][K],
    s16 f16 bits [N].  Returns fp64 [M][N]."""
    X16 = np.ascontiguousarray(X16)
    if X16.dtype == np.float16:
        X16 = X16.view(np.uint16)
    X16 = _c(X16, np.uint16)
    if X16.ndim == 1:
        X16 = X16[None, :]
    s16 = np.ascontiguousarray(s16)
    if s16.dtype == np.float16:
        s16 = s16.view(np.uint16)
    s16 = _c(s16, np.uint16)
    q = _c(q, np.int8)
    M, K = X16.shape
    N = q.shape[0]
    assert q.shape == (N, K) and s16.shape == (N,)
    Y = np.empty((M, N), np.float64)
    _check(_load().qwo_gemv_w8a16_ref64(_p(X16), _p(q), _p(s16), M, N, K, _p(Y), int(nthreads)))
    return Y


def f16_from_f32(x):
    x = _c(x, np.float32).ravel()
    h = np.empty(x.shape, np.uint16)
    _load().qwo_f16_from_f32_n(_p(x), x.size, _p(h))
    return h


def f32_from_f16(h):
    h = np.ascontiguousarray(h)
    if h.dtype == np.float16:
        h = h.view(np.uint16)
    h = _c(h, np.uint16).ravel()
    x = np.empty(h.shape, np.float32)
    _load().qwo_f32_from_f16_n(_p(h), h.size, _p(x))
    return x
