"""Host-side tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before making any HIP call (so they run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_quantized_load_amd as qw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwgemv.h")

if not os.path.exists(qw.LIB_PATH):  # build once if nothing is built
    import __graft_entry__

    __graft_entry__.build()

L = qw.lib()
NULL = ctypes.c_void_p(0)
A = ctypes.c_void_p(0x10000)    # aligned fake device address (never dereferenced)
A2 = ctypes.c_void_p(0x20000)
A3 = ctypes.c_void_p(0x30000)
A4 = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10004)  # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) == 35
    for n in names:
        assert hasattr(L, n), n
        assert n in qw.SIGNATURES, n
    assert sorted(qw.SIGNATURES) == names


def test_packed_sizes():
    # tile layout: 1 KB tiles of 512 k by 4 rows (INT4) or 2 rows (INT8)
    assert L.qw_w4_packed_bytes(18944, 3584) == 18944 * 3584 // 2
    assert L.qw_w8_packed_bytes(27392, 4096) == 27392 * 4096
    assert L.qw_w8_packed_bytes(18944, 3584) == 18944 * 3584
    assert L.qw_w4_packed_bytes(152064, 3584) == 152064 * 3584 // 2
    assert L.qw_w4_packed_bytes(5, 96) == 2 * 1 * 1024
    assert L.qw_w8_packed_bytes(517, 288) == 259 * 1 * 1024
    assert L.qw_w4_packed_bytes(3584, 18944) == 896 * 37 * 1024
    assert L.qw_w4_packed_bytes(0, 64) == 0
    assert L.qw_w4_packed_bytes(8, 48) == 0


def test_status_strings():
    for st in range(8):
        assert L.qw_status_str(st)
    assert L.qw_status_str(99) == b"unknown status"


def test_which_shapes_need_a_workspace():
    # the GEMVs (W4A8 at M == 1, W8A16 at any M) need none
    for (M, N, K) in [(1, 512, 256), (1, 18944, 3584), (1, 3584, 18944), (1, 512, 3584)]:
        assert L.qw_workspace_bytes(0, M, N, K) == 0
    for (M, N, K) in [(1, 512, 256), (4, 27392, 4096), (3, 5, 96), (15, 7, 512), (512, 64, 4096)]:
        assert L.qw_workspace_bytes(1, M, N, K) == 0
    # W4A8 from M == 2 runs on the matrix cores with a workspace
    for (M, N, K) in [(4, 27392, 4096), (3, 5, 96), (15, 7, 512)]:
        assert L.qw_workspace_bytes(0, M, N, K) > 0


def test_skinny_w4a8_workspace_size_and_checks():
    def align(x):
        return (x + 255) // 256 * 256
    for (M, K) in [(16, 4096), (17, 544), (512, 4096), (65535, 3584)]:
        want = align(-(-M // 16) * -(-K // 64) * 1024) + align(4 * M)
        assert L.qw_workspace_bytes(0, M, 27392, K) == want, (M, K)
        assert L.qw_workspace_bytes(1, M, 27392, K) == 0
    # M == 1 needs none; from M == 2 W4A8 needs one
    assert L.qw_workspace_bytes(0, 1, 27392, 4096) == 0
    assert L.qw_workspace_bytes(0, 2, 27392, 4096) == align(4096 // 64 * 1024) + align(8)
    # M >= 2 needs the workspace; validation fails before anything is launched
    assert L.gemv_w4a8(A, A2, A3, 2, 64, 512, A4, NULL, 0, NULL) == qw.QW_ERR_WORKSPACE
    assert L.gemv_w4a8(A, A2, A3, 16, 64, 512, A4, NULL, 0, NULL) == qw.QW_ERR_WORKSPACE
    need = L.qw_workspace_bytes(0, 16, 64, 512)
    assert L.gemv_w4a8(A, A2, A3, 16, 64, 512, A4, A, need - 16, NULL) == qw.QW_ERR_WORKSPACE
    assert L.gemv_w4a8(A, A2, A3, 16, 64, 512, A4, MIS, need, NULL) == qw.QW_ERR_ALIGN


@pytest.mark.parametrize("fn", ["gemv_w4a8", "gemv_w8a16"])
def test_gemv_rejects_bad_arguments(fn):
    f = getattr(L, fn)
    # NULL inputs
    assert f(NULL, A, A, 1, 64, 64, A, NULL, 0, NULL) == qw.QW_ERR_NULL
    # shapes
    for (M, N, K) in [(0, 64, 64), (1, 0, 64), (1, 64, 0), (1, 64, 48), (1, 64, 131072 + 32),
                      (70000, 64, 64), (-1, 64, 64)]:
        assert f(A, A2, A3, M, N, K, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE, (M, N, K)
    # one row of X must fit on chip: K <= 57344 (INT4) or 28672 (INT8)
    kmax = 57344 if fn == "gemv_w4a8" else 28672
    assert f(A, A2, A3, 1, 64, kmax + 32, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE
    # alignment
    assert f(MIS, A2, A3, 1, 64, 64, A4, NULL, 0, NULL) == qw.QW_ERR_ALIGN
    assert f(A, A2, A3, 1, 64, 64, MIS, NULL, 0, NULL) == qw.QW_ERR_ALIGN


@pytest.mark.parametrize("fn", ["qw_gemv_w4a8_tiled", "qw_gemv_w8a16_tiled"])
def test_tiled_rejects_bad_launch_shapes(fn):
    f = getattr(L, fn)
    # (M, N, K, u, nw, nwaves, splitk): bad batch, bad wave count, no waves, register
    # variant for M > 1 or K > 4096, more than 64 row groups per wave; split-K with a
    # bad factor, with the register or eager variant, with 16 waves, or with more than
    # 16 row groups per row run
    for (M, N, K, u, nw, nwaves, sk) in [(1, 64, 4096, 3, 8, 1, 1), (1, 64, 4096, 8, 5, 1, 1),
                                         (1, 64, 4096, 8, 8, 0, 1), (1, 64, 4096, 8, 8, -1, 1),
                                         (2, 64, 4096, 0, 4, 16, 1), (1, 64, 8192, 0, 4, 16, 1),
                                         (1, 1000, 512, 8, 4, 1, 1), (1, 64, 4096, 8, 8, 1, 3),
                                         (1, 64, 4096, 0, 4, 16, 2), (1, 64, 4096, 1, 4, 16, 2),
                                         (1, 64, 4096, 8, 16, 16, 2), (1, 200, 4096, 8, 4, 1, 2),
                                         (1, 64, 4096, 8, 4, 16, 0)]:
        assert f(A, A2, A3, M, N, K, A4, u, nw, nwaves, sk, NULL) == qw.QW_ERR_TILING, \
            (M, N, u, nw, nwaves, sk)
    assert f(A, A2, A3, 1, 64, 4016, A4, 8, 8, 1, 1, NULL) == qw.QW_ERR_SHAPE
    assert f(NULL, A2, A3, 1, 64, 40, A4, 8, 8, 1, 1, NULL) == qw.QW_ERR_NULL
    assert f(MIS, A2, A3, 1, 64, 4096, A4, 8, 8, 1, 1, NULL) == qw.QW_ERR_ALIGN


def test_long_k_w4a8_rejects_bad_arguments_on_the_host():
    """Every check of qw_gemv_w4a8_long_k runs before any launch (no GPU here)."""
    f = L.qw_gemv_w4a8_long_k
    ws = 1 << 20
    M, N, K = 2, 64, 8192  # 16 tiles a row, 16 row groups
    assert f(A, A2, A3, M, N, K, A4, A, ws, 9, 1, NULL) == qw.QW_ERR_TILING   # > 8 waves
    assert f(A, A2, A3, M, N, K, A4, A, ws, 1, 1, NULL) == qw.QW_ERR_TILING   # 16-tile slice
    assert f(A, A2, A3, M, N, K, A4, A, ws, 2, 0, NULL) == qw.QW_ERR_TILING   # no workgroup
    assert f(A, A2, A3, M, N, K, A4, A, ws, 2, 17, NULL) == qw.QW_ERR_TILING  # > row groups
    assert f(A, A2, A3, M, 256, K, A4, A, ws, 2, 1, NULL) == qw.QW_ERR_TILING  # 64 row groups on one
    assert f(NULL, A2, A3, M, N, K, A4, A, ws, 2, 4, NULL) == qw.QW_ERR_NULL
    assert f(MIS, A2, A3, M, N, K, A4, A, ws, 2, 4, NULL) == qw.QW_ERR_ALIGN
    need = L.qw_workspace_bytes(2, M, N, K)
    assert f(A, A2, A3, M, N, K, A4, A, need - 1, 2, 4, NULL) == qw.QW_ERR_WORKSPACE
    assert f(A, A2, A3, M, N, K, A4, NULL, need, 2, 4, NULL) == qw.QW_ERR_WORKSPACE
    assert f(A, A2, A3, M, N, 40, A4, A, ws, 2, 4, NULL) == qw.QW_ERR_SHAPE  # K % 32


@pytest.mark.parametrize("fn", ["qw_gemm_w4a8_mfma", "qw_gemm_w8a16_mfma"])
def test_matrix_core_helpers_reject_bad_launch_shapes(fn):
    f = getattr(L, fn)
    w4 = fn == "qw_gemm_w4a8_mfma"

    def call(X, M, K, nw, mb, nbw, ws=A2, wsb=1 << 20):
        if w4:
            return f(X, A2, A3, M, 64, K, A4, ws, wsb, nw, mb, nbw, NULL)
        return f(X, A2, A3, M, 64, K, A4, nw, mb, nbw, NULL)

    for (nw, mb, nbw) in [(2, 1, 1), (16, 1, 1), (4, 3, 1), (4, 1, 3), (4, 1, 0), (8, 4, 8)]:
        assert call(A, 16, 512, nw, mb, nbw) == qw.QW_ERR_TILING, (nw, mb, nbw)
    if not w4:  # W8A16: at most 2 blocks of rows, and not 8 waves of 2 row blocks
        assert call(A, 16, 512, 4, 4, 1) == qw.QW_ERR_TILING
        assert call(A, 16, 512, 8, 1, 2) == qw.QW_ERR_TILING
    else:  # the workspace is checked
        assert call(A, 16, 512, 4, 1, 1, ws=NULL, wsb=0) == qw.QW_ERR_WORKSPACE
        assert call(A, 16, 512, 4, 1, 1, wsb=100) == qw.QW_ERR_WORKSPACE
        assert L.qw_workspace_bytes(2, 3, 64, 512) == L.qw_workspace_bytes(0, 16, 64, 512)
    assert call(A, 16, 500, 4, 1, 1) == qw.QW_ERR_SHAPE
    assert call(NULL, 16, 512, 4, 1, 1) == qw.QW_ERR_NULL
    assert call(MIS, 16, 512, 4, 1, 1) == qw.QW_ERR_ALIGN


def test_packers_and_helpers_reject_bad_arguments():
    assert L.quantize_pack_w4(NULL, 4, 64, A, A2, NULL) == qw.QW_ERR_NULL
    assert L.quantize_pack_w4(A, 4, 60, A2, A3, NULL) == qw.QW_ERR_SHAPE
    assert L.quantize_pack_w4(MIS, 4, 64, A2, A3, NULL) == qw.QW_ERR_ALIGN
    assert L.quantize_pack_w8(A, 4, 64, A2, NULL, NULL) == qw.QW_ERR_NULL
    assert L.quantize_pack_w8(A, 0, 64, A2, A3, NULL) == qw.QW_ERR_SHAPE
    assert L.quant_act_i8(A, 1, 64, NULL, A2, NULL) == qw.QW_ERR_NULL
    assert L.quant_act_i8(A, 1, 40, A2, A3, NULL) == qw.QW_ERR_SHAPE
    assert L.qw_w4_codes(A, 4, 64, MIS, NULL) == qw.QW_ERR_ALIGN
    assert L.qw_w8_codes(NULL, 4, 64, A, NULL) == qw.QW_ERR_NULL
    assert L.qw_workspace_clear(A, 0, NULL) == qw.QW_OK
    assert L.qw_workspace_clear(NULL, 256, NULL) == qw.QW_ERR_NULL
    assert L.qw_workspace_clear(MIS, 256, NULL) == qw.QW_ERR_ALIGN
    assert L.qw_gemv_w4a8_debug(A, A2, A3, 1, 64, 64, A4, MIS, NULL, NULL, NULL, 0, NULL) \
        == qw.QW_ERR_ALIGN


def test_group_wise_sizes_and_argument_checks():
    # scale layout: per row group, 4 rows x (512 / g) groups x tiles padded to 4
    assert L.qw_w4g_scale_bytes(18944, 3584, 128) == 4736 * 4 * 4 * 8 * 4
    assert L.qw_w4g_scale_bytes(3584, 18944, 128) == 896 * 4 * 4 * 40 * 4
    assert L.qw_w4g_scale_bytes(5, 1056, 32) == 2 * 4 * 16 * 4 * 4
    assert L.qw_w4g_scale_bytes(64, 512, 512) == 16 * 4 * 1 * 4 * 4
    for g in (0, 16, 48, 100, 1024):
        assert L.qw_w4g_scale_bytes(64, 3072, g) == 0, g
    assert L.qw_w4g_scale_bytes(64, 3200, 256) == 0      # K not a multiple of g
    # packer
    assert L.quantize_pack_w4g(NULL, 4, 256, 64, A, A2, NULL) == qw.QW_ERR_NULL
    assert L.quantize_pack_w4g(A, 4, 256, 96, A2, A3, NULL) == qw.QW_ERR_SHAPE
    assert L.quantize_pack_w4g(A, 4, 3200, 512, A2, A3, NULL) == qw.QW_ERR_SHAPE
    assert L.quantize_pack_w4g(A, 4, 256, 64, A2, MIS, NULL) == qw.QW_ERR_ALIGN
    assert L.qw_w4g_scales(A, 4, 256, 33, A2, NULL) == qw.QW_ERR_SHAPE
    # GEMV: M == 1 only, a supported group dividing K, K within the producer-wave shapes
    f = L.gemv_w4a8g
    assert f(NULL, A2, A3, 1, 64, 512, 128, A4, NULL, 0, NULL) == qw.QW_ERR_NULL
    assert f(A, A2, A3, 2, 64, 512, 128, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE
    assert f(A, A2, A3, 1, 64, 512, 48, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE
    assert f(A, A2, A3, 1, 64, 3200, 256, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE
    assert f(A, A2, A3, 1, 64, 32768, 128, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE  # > 24576
    assert f(A, A2, MIS, 1, 64, 512, 128, A4, NULL, 0, NULL) == qw.QW_ERR_ALIGN
    t = L.qw_gemv_w4a8g_tiled
    # only the producer-wave shapes: u 5 with (8, 2) or (4, 4), u 6 with <= 6 tiles a wave
    for (K, u, nw, nwaves, sk) in [(512, 0, 4, 16, 1), (512, 5, 6, 12, 2), (512, 5, 8, 12, 2),
                                   (3584, 6, 8, 256, 3), (18944, 6, 8, 2048, 4),
                                   (28672, 6, 8, 2048, 8)]:
        assert t(A, A2, A3, 1, 64, K, 128, A4, u, nw, nwaves, sk, NULL) == qw.QW_ERR_TILING, \
            (K, u, nw, nwaves, sk)
    # the row-wise tiled entry rejects producer-wave shapes that do not exist
    w4 = L.qw_gemv_w4a8_tiled
    assert w4(A, A2, A3, 1, 64, 512, A4, 5, 8, 8, 3, NULL) == qw.QW_ERR_TILING
    assert w4(A, A2, A3, 2, 64, 512, A4, 5, 8, 8, 2, NULL) == qw.QW_ERR_TILING
    assert w4(A, A2, A3, 1, 64, 32768, A4, 6, 8, 2048, 8, NULL) == qw.QW_ERR_TILING
    assert L.qw_gemv_w8a16_tiled(A, A2, A3, 1, 64, 512, A4, 5, 8, 8, 2, NULL) == qw.QW_ERR_TILING


def test_ablation_entry_points_check_arguments():
    for f in (L.qw_gemv_f16,):
        assert f(NULL, A2, 1, 64, 512, A3, 0, NULL) == qw.QW_ERR_NULL
        assert f(A, A2, 2, 64, 512, A3, 0, NULL) == qw.QW_ERR_SHAPE     # M == 1 only
        assert f(A, A2, 1, 64, 4608, A3, 0, NULL) == qw.QW_ERR_SHAPE    # K <= 4096
        assert f(A, A2, 1, 64, 500, A3, 0, NULL) == qw.QW_ERR_SHAPE
        assert f(A, MIS, 1, 64, 512, A3, 0, NULL) == qw.QW_ERR_ALIGN
        assert f(A, A2, 1, 64, 512, A3, 3, NULL) == qw.QW_ERR_TILING
    g = L.qw_gemv_w4f32
    assert g(A, A2, NULL, 1, 64, 512, A3, 0, NULL) == qw.QW_ERR_NULL
    assert g(A, A2, A4, 3, 64, 512, A3, 0, NULL) == qw.QW_ERR_SHAPE
    assert g(A, A2, MIS, 1, 64, 512, A3, 0, NULL) == qw.QW_ERR_ALIGN
    assert g(A, A2, A4, 1, 64, 512, A3, 8, NULL) == qw.QW_ERR_TILING


def test_index_softmax_checks_and_threshold():
    f = L.index_softmax
    assert f(NULL, 4, 64, 100, 5, 6.6, A2, NULL) == qw.QW_ERR_NULL
    for (rows, Ln, ci, b, c) in [(0, 64, 100, 5, 6.6), (4, 0, 100, 5, 6.6), (4, 16385, 100, 5, 6.6),
                                 (4, 64, 0, 5, 6.6), (4, 64, 100, 3, 6.6), (4, 64, 100, 7, 6.6),
                                 (4, 64, 100, 5, 0.0), (4, 64, 100, 5, -1.0)]:
        assert f(A, rows, Ln, ci, b, c, A2, NULL) == qw.QW_ERR_SHAPE, (rows, Ln, ci, b, c)
    assert f(MIS, 4, 64, 100, 5, 6.6, A2, NULL) == qw.QW_ERR_ALIGN
    assert f(A, 4, 64, 100, 5, 6.6, MIS, NULL) == qw.QW_ERR_ALIGN
    assert L.qw_index_cint(6.6, 128, 0.02, 0.03) == 124451      # 124450.79...
    assert L.qw_index_cint(6.6, 128, 0.0, 0.03) == -1
    assert L.qw_index_cint(6.6, 128, 1e-9, 1e-9) == -1          # beyond int32


def test_index_magic_matches_the_rounded_ratio():
    """The multiply-high table index of the IndexSoftmax kernel: for every c_int and b it
    accepts, (mulhi(2 n D' + c_int, magic) >> shift) equals round(D' n / c_int) half up
    (the integer definition) at D' = 0, c_int, both sides of every half-step and random
    points; outside its bound it declines."""
    rng = np.random.default_rng(7)
    m = ctypes.c_uint32(0)
    sh = ctypes.c_int(0)
    cints = [1, 2, 3, 5, 62, 64, 1000, 124451, 2**20, 3 * 10**6, 2**24 - 1, 2**24, 2**31 - 1]
    cints += [int(v) for v in rng.integers(1, 2**24, size=40)]
    took = 0
    for b in (4, 5, 6):
        n = 2**b - 1
        for ci in cints:
            ok = L.qw_index_magic(ci, b, ctypes.byref(m), ctypes.byref(sh))
            fits = ci < 2**24 and ci * (2 * n + 1) < 2**31
            assert ok == (1 if fits else 0), (ci, b)
            if not ok:
                continue
            took += 1
            mag, s = m.value, sh.value
            ds = {0, ci, ci - 1}
            for k in range(1, n + 1):  # both sides of the half-step boundaries
                t = -(-ci * (2 * k - 1) // (2 * n))
                ds |= {t - 1, t, t + 1}
            ds |= {int(v) for v in rng.integers(0, ci + 1, size=200)}
            for d in ds:
                if not 0 <= d <= ci:
                    continue
                want = (2 * n * d + ci) // (2 * ci)
                got = (((2 * n * d + ci) * mag) >> 32) >> s
                assert got == want, (ci, b, d)
    assert took >= 100
    assert L.qw_index_magic(100, 3, ctypes.byref(m), ctypes.byref(sh)) == 0
    assert L.qw_index_magic(0, 5, ctypes.byref(m), ctypes.byref(sh)) == 0
    assert L.qw_index_magic(100, 5, NULL, ctypes.byref(sh)) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(qw, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(qw, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        qw.lib()


def test_stream_read_and_device_status_check_arguments_on_the_host():
    sink = A2
    assert L.qw_stream_read(NULL, 1024, sink, 0, 0, 0, NULL) == qw.QW_ERR_NULL
    assert L.qw_stream_read(A, 1024, NULL, 0, 0, 0, NULL) == qw.QW_ERR_NULL
    assert L.qw_stream_read(A, 0, sink, 0, 0, 0, NULL) == qw.QW_ERR_SHAPE
    assert L.qw_stream_read(A, 1000, sink, 0, 0, 0, NULL) == qw.QW_ERR_SHAPE
    assert L.qw_stream_read(MIS, 1024, sink, 0, 0, 0, NULL) == qw.QW_ERR_ALIGN
    for bad in [(3, 1, 4), (8, -1, 4), (8, 1, 3), (32, 1, 4), (8, 70000, 4)]:
        assert L.qw_stream_read(A, 1024, sink, *bad, NULL) == qw.QW_ERR_TILING, bad
    # one workgroup's share would need a buffer resource of 2 GiB or more
    assert L.qw_stream_read(A, 1 << 31, sink, 8, 1, 4, NULL) == qw.QW_ERR_SHAPE
    assert L.qw_device_status(NULL, 0) == qw.QW_ERR_NULL


def test_noalloc_w4a8_checks_arguments_and_its_limit_on_the_host():
    f = L.gemv_w4a8_noalloc
    assert f(NULL, A2, A3, 2, 64, 512, A4, NULL) == qw.QW_ERR_NULL
    assert f(A, A2, A3, 2, 64, 500, A4, NULL) == qw.QW_ERR_SHAPE
    assert f(A, A2, A3, 0, 64, 512, A4, NULL) == qw.QW_ERR_SHAPE
    # 512 rows fit the 8 MiB array up to K = 16320; 16384 does not
    assert L.qw_workspace_bytes(0, 512, 64, 16320) <= 8 << 20 < L.qw_workspace_bytes(0, 512, 64, 16384)
    assert f(A, A2, A3, 512, 64, 16384, A4, NULL) == qw.QW_ERR_WORKSPACE
    assert f(A, A2, A3, 4096, 64, 4096, A4, NULL) == qw.QW_ERR_WORKSPACE


def test_tile_routing_choices():
    """The tiled-GEMM routing (qw_tile_variant, the choice gemv_w4a8 / gemv_w8a16 make on
    their matrix-core path) for the 256-CU model used without a visible device: the
    documented choices and the shapes the GPU routing test relies on."""
    v = L.qw_tile_variant
    # W8A16 on 4096 -> 27392: 128 x 32 tiles from 12 rows, then by the tile model
    assert [v(8, M, 27392) for M in (9, 11, 12, 16, 32)] == [-1, -1, 8, 8, 8]
    assert [v(8, M, 27392) for M in (33, 64, 128, 256, 512)] == [7, 7, 3, 1, 0]
    # W4A8: 128 x 32 tiles from 20 rows, the tile model from 33
    assert [v(4, M, 27392) for M in (16, 19, 20, 32)] == [-1, -1, 8, 8]
    assert [v(4, M, 27392) for M in (64, 128, 256, 512)] == [7, 2, 1, 0]
    # fewer than 128 tiles of 128 x 32 below 33 rows: the balanced kernels
    assert v(8, 16, 9000) == -1 and v(8, 24, 9000) == -1 and v(4, 24, 9000) == -1
    assert v(8, 16, 16256) == -1 and v(8, 16, 16257) == 8
    # 4096 -> 9000 from 33 rows, 3584 -> 18944 at 96 rows
    assert [v(8, M, 9000) for M in (48, 64, 96, 128)] == [8, 8, 8, 7]
    assert v(8, 96, 18944) == 8 and v(4, 96, 18944) == 8
    # the default-path shapes of the GPU routing test
    routed = [(40, 9000), (40, 20000), (70, 20000), (70, 34000), (520, 20000), (70, 6000),
              (70, 9000), (130, 34000), (520, 6000), (40, 3000), (24, 9000), (24, 20000)]
    assert [v(8, M, N) for M, N in routed] == [8, 7, 8, 1, 0, 8, 8, 0, 3, -1, -1, 8]
    assert [v(4, M, N) for M, N in routed] == [8, 7, 8, 1, 0, 8, 8, 0, 2, -1, -1, 8]
    # at least 96 tiles: narrow outputs stay on the balanced kernels at any M
    assert v(8, 64, 3584) == -1 and v(4, 64, 3584) == -1
    assert v(3, 64, 27392) == -1 and v(8, 0, 27392) == -1
