"""Parity of the INT4 page's two ablation kernels with the CPU oracle (section 速度结果
of "Jetson Orin AGX 上的 INT4 量化推理实践"): the FP16 GEMV and weight-only INT4 with float
activations.

Bars: FP16 within relative L2 error 1e-3 of the fp64 value (its f16 output rounding alone
is about 3e-4, as for W8A16); weight-only INT4 within the fp32 multiply-add bound
(K + 2) * 2^-24 * s * sum_k |q x| of the fp64 value, per element.  Every rows-per-wave
choice adds a row's products in the same order (same bits).  On activations that are
integers in [-127, 127] with a 127 present, the float-unpack path and the W4A8 integer
path give the same bits (every partial sum is an exact fp32 integer).
"""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import oracle
import workloads as wl

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


SHAPES = [(18944, 3584), (512, 3584), (3584, 3584), (1000, 1056), (37, 96), (4101, 4096)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_fp16_gemv(N, K):
    print("fp16 GEMV", N, K, flush=True)
    W16 = wl.weights(81, 1, N, K).astype(np.float16)
    X16 = wl.activations(81, 2, 1, K, dtype=np.float16)
    y64 = oracle.gemv_f16_ref64(X16, W16, nthreads=oracle.num_threads())
    Xd, Wd = dev(X16), dev(W16)
    first = None
    for rpw in (0, 1, 2, 4):
        y = host(qw.gemv_f16(Xd, Wd, rows_per_wave=rpw)).astype(np.float64)
        err = np.linalg.norm(y - y64) / np.linalg.norm(y64)
        assert err <= 1e-3, (rpw, err)
        first = y if first is None else first
        assert np.array_equal(y, first), rpw


@pytest.mark.parametrize("N,K", SHAPES)
def test_weight_only_int4_float_unpack(N, K):
    print("weight-only INT4 float", N, K, flush=True)
    W = wl.weights(82, 1, N, K, outlier_rows=True)
    X = wl.activations(82, 2, 1, K, outlier_channels=4)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q, so = oracle.quant_w4(W)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    Y, Y64 = oracle.gemv_w4f32(X, q, so, nthreads=oracle.num_threads())
    bound = oracle.w4f32_bound(X, q, so) + 2.0 ** -140
    assert np.all(np.abs(Y - Y64) <= bound)
    Xd = dev(X)
    first = None
    for rpw in (0, 1, 2, 4):
        y = host(qw.gemv_w4f32(Xd, Wq, s, rows_per_wave=rpw))
        assert np.all(np.abs(y.astype(np.float64) - Y64) <= bound), rpw
        first = y if first is None else first
        assert np.array_equal(y.view(np.uint32), first.view(np.uint32)), rpw


def test_float_unpack_equals_integer_path_on_integer_activations():
    N, K = 4608, 3584
    W = wl.weights(83, 1, N, K, outlier_rows=True)
    Wq, s = qw.quantize_pack_w4(dev(W))
    X = np.random.default_rng(83).integers(-127, 128, size=(1, K)).astype(np.float32)
    X[0, 11] = 127.0
    yf = host(qw.gemv_w4f32(dev(X), Wq, s))
    yi = host(qw.gemv_w4a8(dev(X), Wq, s))
    assert np.array_equal(yf.view(np.uint32), yi.view(np.uint32))
