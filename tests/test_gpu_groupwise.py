"""Parity of the group-wise W4A8 path (one INT4 scale per output row and group of g
consecutive k) with the CPU oracle, through the C ABI, on an MI355X.

Bars: INT4 codes and fp32 group scales bit-exact; outputs within the fp32 summation
bound (K/g + 2) * 2^-24 * sum_t |acc_t * s_t| * |a| of the exact value, computed in fp64
from the oracle's exact per-group dots (the kernel adds the groups in its own order; the
bound holds for any order).  With one group per row (g == K) the output equals the
row-wise GEMV bit for bit.
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


def say(*a):
    print(*a, flush=True)


def pack_and_check(W, g):
    """GPU group-wise pack of W; codes and decoded scales equal the oracle's bit for bit."""
    N, K = W.shape
    Wq, s = qw.quantize_pack_w4g(dev(W), g)
    q_o, s_o = oracle.quant_w4g(W, g)
    assert np.array_equal(host(qw.w4_codes(Wq, N, K)), q_o)
    assert np.array_equal(host(qw.w4g_scales(s, N, K, g)).view(np.uint32), s_o.view(np.uint32))
    return Wq, s, q_o, s_o


def check_y(y, ref, s_o):
    """y within the summation bound of the fp64 value; the oracle's own Y too."""
    y64, bound = oracle.w4a8g_ref64(ref["accg"], s_o, ref["a"])
    bound = bound + 2.0 ** -140
    err = np.abs(np.asarray(y, np.float64) - y64)
    assert np.all(err <= bound), float((err / bound).max())
    assert np.all(np.abs(ref["Y"] - y64) <= bound)


# (N, K, g): Qwen-7B-shaped gate/up, down (K split), q/o, k/v and q|k|v; ragged N and K
# (K not a multiple of 512, so the last tile holds fewer groups); the largest group
GROUP_SHAPES = [(18944, 3584, 128), (3584, 18944, 128), (3584, 3584, 64), (512, 3584, 32),
                (4608, 3584, 256), (1000, 1056, 32), (333, 4640, 32), (8200, 2048, 512),
                (37, 96, 32)]


@pytest.mark.parametrize("N,K,g", GROUP_SHAPES)
def test_group_wise_gemv_matches_oracle(N, K, g):
    say("group-wise W4A8 N", N, "K", K, "g", g)
    W = wl.weights(71, 1, N, K, outlier_rows=True)
    X = wl.activations(71, 2, 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_and_check(W, g)
    ref = oracle.gemv_w4a8g(X, q_o, s_o, g, nthreads=oracle.num_threads())
    Xd = dev(X)
    y = host(qw.gemv_w4a8g(Xd, Wq, s, N, g))
    check_y(y, ref, s_o)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("N,K,g", [(8200, 3584, 128), (1000, 1056, 32), (333, 4608, 64),
                                   (3584, 18944, 256), (37, 12288, 512)])
def test_group_wise_every_launch_shape(N, K, g):
    """Every producer-wave launch shape the group-wise kernels exist for gives outputs
    within the bar; without a K split, the workgroup count does not change the order in
    which a row's groups are added (same bits)."""
    say("group-wise launch shapes N", N, "K", K, "g", g)
    W = wl.weights(72, 1, N, K, outlier_rows=True)
    X = wl.activations(72, 2, 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_and_check(W, g)
    ref = oracle.gemv_w4a8g(X, q_o, s_o, g, nthreads=oracle.num_threads())
    Xd = dev(X)
    nrg, cg = -(-N // 4), -(-K // 512)
    tried = 0
    if cg <= 8:
        for (nw, P) in ((8, 2), (4, 4)):
            first = None
            for blocks in (1, 7, 64, 256):
                y = host(qw.gemv_w4a8g_tiled(Xd, Wq, s, N, g, 5, nw, blocks * nw, P))
                check_y(y, ref, s_o)
                # the workgroup split does not change a row's summation order
                first = y if first is None else first
                assert np.array_equal(y.view(np.uint32), first.view(np.uint32)), (nw, P, blocks)
                tried += 1
    for S in (2, 4, 8):
        if -(-cg // S) > 6:
            continue
        for blocks in sorted({-(-nrg // 16), 64, 256}):
            if -(-nrg // blocks) > 16:
                continue
            y = host(qw.gemv_w4a8g_tiled(Xd, Wq, s, N, g, 6, 8, blocks * 8, S))
            check_y(y, ref, s_o)
            tried += 1
    assert tried >= 3
    with pytest.raises(qw.QWError):
        qw.gemv_w4a8g_tiled(Xd, Wq, s, N, g, 5, 6, 12, 2)


def test_one_group_per_row_equals_row_wise_bit_for_bit():
    N, K = 3000, 512
    W = wl.weights(73, 1, N, K, outlier_rows=True)
    X = wl.activations(73, 2, 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_and_check(W, 512)
    Wr, sr = qw.quantize_pack_w4(dev(W))
    assert np.array_equal(host(Wq), host(Wr))
    assert np.array_equal(host(qw.w4g_scales(s, N, K, 512))[:, 0].view(np.uint32),
                          host(sr).view(np.uint32))
    yg = host(qw.gemv_w4a8g(dev(X), Wq, s, N, 512))
    yr = host(qw.gemv_w4a8(dev(X), Wr, sr))
    assert np.array_equal(yg.view(np.uint32), yr.view(np.uint32))


def test_group_wise_packer_rejects_non_finite_and_zero_groups():
    W = wl.weights(74, 1, 64, 1024)
    W[7, 300:428] = 0.0  # spans two groups of 128 partly, group 3 (384..511) partly
    W[9, 128:256] = 0.0  # exactly group 1 of row 9
    Wq, s, q_o, s_o = pack_and_check(W, 128)
    assert host(qw.w4g_scales(s, 64, 1024, 128))[9, 1] == 0
    W[5, 17] = np.inf
    with pytest.raises(qw.QWError) as e:
        qw.quantize_pack_w4g(dev(W), 128)
    assert e.value.status == qw.QW_ERR_NONFINITE


def test_group_wise_graph_replays_match_eager():
    N, K, g = 4608, 3584, 128
    W = wl.weights(75, 1, N, K)
    X = wl.activations(75, 2, 1, K)
    Wq, s, q_o, s_o = pack_and_check(W, g)
    Xd = dev(X)
    Y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    eager = host(qw.gemv_w4a8g(Xd, Wq, s, N, g)).copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qw.gemv_w4a8g(Xd, Wq, s, N, g, out=Y)
    for _ in range(4):
        Y.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        assert np.array_equal(host(Y).view(np.uint32), eager.view(np.uint32))
