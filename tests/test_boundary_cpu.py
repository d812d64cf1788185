"""Host-side tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before making any HIP call (so they run without a GPU)."""
import ctypes
import os
import re

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
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
        assert n in qw.SIGNATURES, n


def test_packed_sizes():
    assert L.qw_w4_packed_bytes(18944, 3584) == 18944 * 1792
    assert L.qw_w8_packed_bytes(27392, 4096) == 27392 * 4096
    assert L.qw_w4_packed_bytes(0, 64) == 0


def test_status_strings():
    for st in range(8):
        assert L.qw_status_str(st)
    assert L.qw_status_str(99) == b"unknown status"


def test_workspace_sizes_are_aligned():
    for op in (0, 1):
        for (M, N, K) in [(1, 512, 256), (1, 18944, 3584), (1, 3584, 18944), (4, 27392, 4096),
                          (1, 512, 3584), (3, 5, 96)]:
            b = L.qw_workspace_bytes(op, M, N, K)
            assert b % 256 == 0
            if b:
                assert b >= M * N * 4
    assert L.qw_workspace_bytes(0, 1, 512, 33) == 0   # bad shape -> 0
    assert L.qw_workspace_bytes(7, 1, 512, 256) == 0  # bad op -> 0


@pytest.mark.parametrize("fn", ["gemv_w4a8", "gemv_w8a16"])
def test_gemv_rejects_bad_arguments(fn):
    f = getattr(L, fn)
    # NULL inputs
    assert f(NULL, A, A, 1, 64, 64, A, NULL, 0, NULL) == qw.QW_ERR_NULL
    # shapes
    for (M, N, K) in [(0, 64, 64), (1, 0, 64), (1, 64, 0), (1, 64, 48), (1, 64, 131072 + 32),
                      (70000, 64, 64), (-1, 64, 64)]:
        assert f(A, A2, A3, M, N, K, A4, NULL, 0, NULL) == qw.QW_ERR_SHAPE, (M, N, K)
    # alignment
    assert f(MIS, A2, A3, 1, 64, 64, A4, NULL, 0, NULL) == qw.QW_ERR_ALIGN
    assert f(A, A2, A3, 1, 64, 64, MIS, NULL, 0, NULL) == qw.QW_ERR_ALIGN


@pytest.mark.parametrize("fn,op", [("gemv_w4a8", 0), ("gemv_w8a16", 1)])
def test_gemv_rejects_missing_workspace(fn, op):
    f = getattr(L, fn)
    # find a shape for which the built-in tiling splits K and so needs a workspace
    for (M, N, K) in [(1, 512, 3584), (1, 64, 4096), (1, 3584, 18944), (1, 16, 8192)]:
        need = L.qw_workspace_bytes(op, M, N, K)
        if need:
            break
    assert need > 0
    assert f(A, A2, A3, M, N, K, A4, NULL, 0, NULL) == qw.QW_ERR_WORKSPACE
    assert f(A, A2, A3, M, N, K, A4, A, need - 256, NULL) == qw.QW_ERR_WORKSPACE


def test_tiled_rejects_bad_tilings():
    f = L.qw_gemv_w4a8_tiled
    for (cpl, gb, rpw) in [(3, 4, 16), (2, 3, 24), (2, 4, 10), (2, 4, 0), (4, 8, 32)]:
        assert f(A, A2, A3, 1, 64, 256, A4, NULL, 0, cpl, gb, rpw, NULL) == qw.QW_ERR_TILING
    # MT*CPL > 8: M=8 (mt 8) with cpl 2
    assert f(A, A2, A3, 8, 64, 256, A4, NULL, 0, 2, 1, 4, NULL) == qw.QW_ERR_TILING
    assert L.qw_tiled_workspace_bytes(0, 1, 64, 256, 3, 4, 16) == 0


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


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(qw, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(qw, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        qw.lib()
