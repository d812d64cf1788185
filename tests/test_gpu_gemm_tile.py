"""The tiled matrix-core GEMM (one workgroup per output tile of 64 to 256 rows of W by
64 to 256 rows of X, staged through LDS by direct loads, every variant) against the
oracle, on an MI355X.

W8A16 (ChatGLM2-6B W8A16 write-up, section 4): within relative L2 1e-3 of the fp64
dequantize-then-multiply reference and per element within half an f16 ulp plus the
fp32 summation bound.  W4A8 ("Jetson Orin AGX 上的 INT4 量化推理实践", sections 当前实现方式
and 正确方向): the oracle's outputs bit for bit (exact int32 sums, the fixed epilogue).  Shapes: the top of the skinny-GEMM sweep (512 and 64 rows on
4096 -> 27392, checked on sampled rows of W), and ragged M, N and K (a partial tile in
each direction, K % 64 == 32, fewer rows than one tile)."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import oracle
import workloads as wl
from bounds import check_w8a16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    qw.lib()
    yield


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


VARIANTS = tuple(range(9))
SHAPES = [(130, 300, 1056), (64, 128, 4096), (1, 96, 512), (257, 1000, 2080), (300, 37, 96),
          (65, 4100, 3584), (200, 513, 544), (17, 2050, 18944)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a16_tile_every_variant(M, N, K):
    print("w8a16 tile", M, N, K, flush=True)
    W = wl.weights(1500 + M, 1, N, K, outlier_rows=N >= 100)
    W[min(3, N - 1)] = 0.0  # a zero row
    X16 = wl.activations(1500 + M, 2, M, K, outlier_channels=4).astype(np.float16)
    X16[M // 2] = 0  # a zero row of X
    Wq, s16 = qw.quantize_pack_w8(dev(W))
    q8, s16_o = oracle.quant_w8(W)
    assert np.array_equal(host(s16).view(np.uint16), s16_o)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    Xd = dev(X16)
    bad = []
    for v in VARIANTS:
        buf = torch.full((M * N + 64,), float("nan"), dtype=torch.float16, device="cuda")
        Y = buf[:M * N].view(M, N)
        qw.gemm_w8a16_tile(Xd, Wq, s16, v, out=Y)
        y = host(Y)
        try:
            assert np.all(np.isfinite(y.astype(np.float32)))
            assert np.all(np.isnan(host(buf[M * N:]).astype(np.float32)))  # nothing past Y
            check_w8a16(y, X16, q8, s16_o, y64)
            assert not np.any(y[M // 2]) and not np.any(y[:, min(3, N - 1)])
        except AssertionError:
            bad.append(v)
    assert not bad, "variants %s" % bad


@pytest.mark.parametrize("M", [64, 512])
def test_w8a16_tile_sweep_shape_sampled(M):
    c = wl.SKINNY
    K, N = c["K"], c["N"]
    print("w8a16 tile sweep shape", M, K, N, flush=True)
    W = wl.weights(c["seed"], 1, N, K, outlier_rows=True)
    X16 = wl.activations(c["seed"], 2, M, K, outlier_channels=4).astype(np.float16)
    Wq, s16 = qw.quantize_pack_w8(dev(W))
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(0, 160), np.arange(N - 160, N),
                                     rng.choice(N, 400, replace=False)]))
    q8, s16_o = oracle.quant_w8(W[rows])
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    ridx = torch.as_tensor(rows, device="cuda")
    Xd = dev(X16)
    for v in VARIANTS:
        Y = qw.gemm_w8a16_tile(Xd, Wq, s16, v)
        check_w8a16(host(Y[:, ridx]), X16, q8, s16_o, y64)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a8_tile_every_variant(M, N, K):
    print("w4a8 tile", M, N, K, flush=True)
    W = wl.weights(1600 + M, 1, N, K, outlier_rows=N >= 100)
    W[min(3, N - 1)] = 0.0
    X = wl.activations(1600 + M, 2, M, K, outlier_channels=4)
    X[M // 2] = 0.0
    Wq, s = qw.quantize_pack_w4(dev(W))
    q, s_o = oracle.quant_w4(W)
    assert np.array_equal(host(s).view(np.uint32), s_o.view(np.uint32))
    ref = oracle.gemv_w4a8(X, q, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    ws = torch.empty(int(qw.lib().qw_workspace_bytes(2, M, N, K)), dtype=torch.uint8, device="cuda")
    bad = []
    for v in VARIANTS:
        buf = torch.full((M * N + 64,), float("nan"), device="cuda")
        Y = buf[:M * N].view(M, N)
        qw.gemm_w4a8_tile(Xd, Wq, s, v, workspace=ws, out=Y)
        y = host(Y)
        if not (np.all(np.isnan(host(buf[M * N:]))) and np.array_equal(y.view(np.uint32), ref["Y"].view(np.uint32))):
            bad.append(v)
    assert not bad, "variants %s" % bad


@pytest.mark.parametrize("M", [64, 512])
def test_w4a8_tile_sweep_shape_sampled(M):
    c = wl.SKINNY
    K, N = c["K"], c["N"]
    print("w4a8 tile sweep shape", M, K, N, flush=True)
    W = wl.weights(c["seed"], 1, N, K, outlier_rows=True)
    X = wl.activations(c["seed"], 2, M, K, outlier_channels=4)
    Wq, s = qw.quantize_pack_w4(dev(W))
    rng = np.random.default_rng(M + 1)
    rows = np.unique(np.concatenate([np.arange(0, 160), np.arange(N - 160, N),
                                     rng.choice(N, 400, replace=False)]))
    q, s_o = oracle.quant_w4(W[rows])
    ref = oracle.gemv_w4a8(X, q, s_o, nthreads=oracle.num_threads())
    ridx = torch.as_tensor(rows, device="cuda")
    Xd = dev(X)
    for v in VARIANTS:
        Y = qw.gemm_w4a8_tile(Xd, Wq, s, v)
        assert np.array_equal(host(Y[:, ridx]).view(np.uint32), ref["Y"].view(np.uint32)), v


# The default entry points route to the tiled GEMM from 33 rows of X where the output has
# at least 96 tiles, choosing the variant by a model of the tiles on the busiest CU, and
# from 12 (W8A16) or 20 (W4A8) rows where there are at least 128 tiles of 128 x 32.  On
# the 256-CU MI355X these shapes reach variants 8, 7, 8, 1, 0, 8, 8, 0, 3 (W4A8: 2), the
# balanced kernels (3000 rows of W at 40 rows, 9000 at 24), and variant 8 at 24 rows.
# Checked on sampled rows of W.
ROUTED = [(40, 9000, 1056), (40, 20000, 544), (70, 20000, 2080), (70, 34000, 512), (520, 20000, 512),
          (70, 6000, 4096), (70, 9000, 1056), (130, 34000, 512), (520, 6000, 544), (40, 3000, 18944),
          (24, 9000, 1056), (24, 20000, 1056)]


@pytest.mark.parametrize("M,N,K", ROUTED)
def test_default_paths_through_the_tiled_gemm(M, N, K):
    print("default routed", M, N, K, flush=True)
    W = wl.weights(1700 + M, 1, N, K, outlier_rows=True)
    X = wl.activations(1700 + M, 2, M, K, outlier_channels=4)
    X[M // 3] = 0.0
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(N - 70, N),
                                     rng.choice(N, 300, replace=False)]))
    ridx = torch.as_tensor(rows, device="cuda")
    Wd = dev(W)
    Wq, s = qw.quantize_pack_w4(Wd)
    q, s_o = oracle.quant_w4(W[rows])
    ref = oracle.gemv_w4a8(X, q, s_o, nthreads=oracle.num_threads())
    Y = qw.gemv_w4a8(dev(X), Wq, s, workspace=qw.make_workspace("w4a8", M, N, K))
    assert np.array_equal(host(Y[:, ridx]).view(np.uint32), ref["Y"].view(np.uint32))
    del Wq, s
    X16 = X.astype(np.float16)
    Wq8, s16 = qw.quantize_pack_w8(Wd)
    q8, s16_o = oracle.quant_w8(W[rows])
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    y = qw.gemv_w8a16(dev(X16), Wq8, s16)
    check_w8a16(host(y[:, ridx]), X16, q8, s16_o, y64)
    assert not np.any(host(y[M // 3]))
