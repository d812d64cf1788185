"""gemv_w4a8_noalloc on an MI355X, through the C ABI: the allocation-free form of
gemv_w4a8 (its activation codes and scales in the library's fixed per-GPU scratch array
instead of a caller's workspace) gives gemv_w4a8's output bits on two calls in a row, the
second with a smaller input, so what the first call left in the array does not leak into
the second; a shape beyond the array is rejected with QW_ERR_WORKSPACE."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    qw.lib()
    yield


def _case(seed, M, N, K):
    W = torch.from_numpy(wl.weights(seed, 1, N, K, outlier_rows=True)).cuda()
    Wq, s = qw.quantize_pack_w4(W)
    X = torch.from_numpy(wl.activations(seed, 2, M, K, outlier_channels=4)).cuda()
    return X, Wq, s


@pytest.mark.parametrize("first,second", [
    ((512, 27392, 4096), (64, 3000, 3584)),   # matrix-core path, then a smaller one
    ((16, 3584, 18944), (3, 512, 18944)),     # long-K kernels (row-major codes)
    ((40, 1000, 1056), (2, 100, 512)),
    ((2, 4096, 4096), (1, 4096, 4096)),       # down to one row (no scratch used)
])
def test_noalloc_equals_gemv_w4a8_on_two_calls(first, second):
    outs = []
    for i, (M, N, K) in enumerate((first, second)):
        print("noalloc call", i, M, N, K, flush=True)
        X, Wq, s = _case(1400 + i, M, N, K)
        Y = torch.full((M, N), float("nan"), device="cuda")
        qw.gemv_w4a8_noalloc(X, Wq, s, out=Y)
        outs.append((Y, X, Wq, s))
    for (Y, X, Wq, s) in outs:
        M, K = X.shape
        ref = qw.gemv_w4a8(X, Wq, s, workspace=qw.make_workspace("w4a8", M, s.shape[0], K))
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))


def test_noalloc_rejects_shapes_beyond_its_array():
    M, N, K = 512, 64, 16384
    X, Wq, s = _case(1410, M, N, K)
    with pytest.raises(qw.QWError) as e:
        qw.gemv_w4a8_noalloc(X, Wq, s)
    assert e.value.status == qw.QW_ERR_WORKSPACE
