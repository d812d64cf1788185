"""Parity of the HIP path with the CPU oracle, through the C ABI, on an MI355X.

Bars: INT4/INT8 codes, packed bytes, fp32/f16 scales and int32 accumulators are
bit-exact; W4A8 outputs within 1e-6 relative error per element; W8A16 outputs within
1e-3 relative L2 error of the fp64 dequantize-then-multiply reference.  Inputs are
the seeded synthetic workloads of the ``workloads`` module.  Full-size shapes that
the oracle cannot finish in seconds are checked on sampled output rows.
"""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import oracle
import workloads as wl
from bounds import check_w8a16, rel_l2  # noqa: F401

pytestmark = pytest.mark.gpu

W4A8_RTOL = 1e-6
W8A16_RL2 = 1e-3


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


def routed_to_tile(bits, M, N):
    """Whether gemv_w4a8 / gemv_w8a16 send M rows to the tiled GEMM (its routing rule):
    from 33 rows where some variant has at least 96 tiles (the most tiles: 64 x 64 or
    128 x 32), below that from 12 (W8A16) or 20 (W4A8) rows where there are at least
    128 tiles of 128 x 32."""
    if M < 33:
        return M >= (12 if bits == 8 else 20) and -(-N // 128) >= 128
    return max(-(-N // 64) * -(-M // 64), -(-N // 128) * -(-M // 32)) >= 96


def say(*a):
    print(*a, flush=True)


def assert_w4a8_close(y, yo):
    y = np.asarray(y, np.float64)
    yo = np.asarray(yo, np.float64)
    zero = yo == 0
    assert np.all(y[zero] == 0)
    rel = np.abs(y[~zero] - yo[~zero]) / np.abs(yo[~zero])
    assert rel.size == 0 or rel.max() <= W4A8_RTOL, rel.max()


def tile_layout(canon, N, R):
    """Canonical packed rows [N][row_bytes] -> the library's tile layout: 1 KB tiles of
    R rows x 512 k, i.e. R rows x (64 / R) chunks of 16 bytes, R = 4 for INT4 and 2 for
    INT8; tiles row group by row group, k order inside; zero padding past N and K."""
    L = 64 // R
    row_bytes = canon.shape[1]
    cg, nrg = -(-row_bytes // (16 * L)), -(-N // R)
    pad = np.zeros((nrg * R, cg * L * 16), np.uint8)
    pad[:N, :row_bytes] = canon
    return pad.reshape(nrg, R, cg, L, 16).transpose(0, 2, 1, 3, 4).reshape(-1)


def pack_w4_and_check(W, rows=None):
    """GPU pack of W; compares the packed bytes (whole matrix) or the decoded codes (on
    `rows` only when given) and the scales with the oracle.  Returns (Wq, s, q, s)."""
    N, K = W.shape
    Wq, s = qw.quantize_pack_w4(dev(W))
    Wsub = W if rows is None else W[rows]
    q_o, s_o = oracle.quant_w4(Wsub)
    if rows is None:
        assert np.array_equal(host(s).view(np.uint32), s_o.view(np.uint32))
        assert np.array_equal(host(Wq), tile_layout(oracle.pack_w4(q_o), N, 4))
    else:
        ridx = torch.as_tensor(rows, device="cuda")
        assert np.array_equal(host(s[ridx]).view(np.uint32), s_o.view(np.uint32))
        assert np.array_equal(host(qw.w4_codes(Wq, N, K)[ridx]), q_o)
    return Wq, s, q_o, s_o


# ------------------------------------------------------------------ config 0 --

def test_tiny_w4a8_config_bit_exact():
    M, K, N = 1, 256, 512
    say("tiny W4A8 seed 0", M, K, N)
    W = wl.weights(0, wl.tensor_id("tiny", 0), N, K)
    X = wl.activations(0, wl.tensor_id("tiny", 1), M, K)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    codes = host(qw.w4_codes(Wq, N, K))
    assert np.array_equal(codes, q_o)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    ws = None  # no shape needs a workspace
    out = qw.gemv_w4a8_debug(dev(X), Wq, s, workspace=ws)
    assert np.array_equal(host(out["xq"]), ref["xq"])
    assert np.array_equal(host(out["a"]).view(np.uint32), ref["a"].view(np.uint32))
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert_w4a8_close(host(out["Y"]), ref["Y"])
    # the production entry point, into a NaN-poisoned output with guard canaries
    buf = torch.full((M * N + 64,), float("nan"), device="cuda")
    buf[M * N:] = 12345.0
    Y = buf[:M * N].view(M, N)
    qw.gemv_w4a8(dev(X), Wq, s, workspace=ws, out=Y)
    bh = host(buf)
    assert np.all(bh[M * N:] == 12345.0)
    assert np.array_equal(bh[:M * N].reshape(M, N), host(out["Y"]))
    if ws is not None:
        assert not host(ws).any(), "workspace must be left zero-filled"


def test_quant_act_matches_oracle_and_fused_prologue():
    for (M, K, seed) in [(1, 256, 0), (1, 3584, 1), (4, 4096, 4), (3, 18944, 5), (2, 32, 6)]:
        say("quant_act", M, K)
        X = wl.activations(seed, 99, M, K, outlier_channels=4 if K >= 64 else 0)
        if M > 1:
            X[1] = 0.0  # an all-zero row
        xq, a = qw.quant_act_i8(dev(X))
        xq_o, a_o = oracle.quant_act_i8(X)
        assert np.array_equal(host(xq), xq_o)
        assert np.array_equal(host(a).view(np.uint32), a_o.view(np.uint32))
        N = 64
        W = wl.weights(seed, 98, N, K)
        Wq, s = qw.quantize_pack_w4(dev(W))
        out = qw.gemv_w4a8_debug(dev(X), Wq, s, workspace=qw.make_workspace("w4a8", M, N, K))
        assert np.array_equal(host(out["xq"]), xq_o)
        assert np.array_equal(host(out["a"]).view(np.uint32), a_o.view(np.uint32))


# ------------------------------------------------------------------ config 1 --

@pytest.mark.parametrize("name,K,N", wl.QWEN7B_LINEARS)
def test_qwen7b_linear_w4a8(name, K, N):
    seed = wl.QWEN7B_W4A8["seed"]
    say("qwen7b W4A8", name, K, N)
    W = wl.weights(seed, wl.tensor_id(name, 0), N, K, outlier_rows=True)
    X = wl.activations(seed, wl.tensor_id(name, 1), 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    out = qw.gemv_w4a8_debug(dev(X), Wq, s, workspace=qw.make_workspace("w4a8", 1, N, K))
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert_w4a8_close(host(out["Y"]), ref["Y"])
    Y = qw.gemv_w4a8(dev(X), Wq, s, workspace=qw.make_workspace("w4a8", 1, N, K))
    assert_w4a8_close(host(Y), ref["Y"])


# ------------------------------------------------------------------ config 2 --

def pack_w8_and_check(W, rows=None):
    N, K = W.shape
    Wq, s16 = qw.quantize_pack_w8(dev(W))
    Wsub = W if rows is None else W[rows]
    q_o, s16_o = oracle.quant_w8(Wsub)
    if rows is None:
        assert np.array_equal(host(s16).view(np.uint16), s16_o)
        assert np.array_equal(host(Wq), tile_layout(q_o.view(np.uint8), N, 2))
    else:
        ridx = torch.as_tensor(rows, device="cuda")
        assert np.array_equal(host(s16[ridx]).view(np.uint16), s16_o)
        assert np.array_equal(host(qw.w8_codes(Wq, N, K)[ridx]), q_o)
    return Wq, s16, q_o, s16_o


def _w8a16_case(seed, tid_w, tid_x, M, N, K, rows=None):
    W = wl.weights(seed, tid_w, N, K)
    X16 = wl.activations(seed, tid_x, M, K, dtype=np.float16)
    Wq, s16, q_o, s16_o = pack_w8_and_check(W, rows)
    y = qw.gemv_w8a16(dev(X16), Wq, s16)
    y = host(y if rows is None else y[:, torch.as_tensor(rows, device="cuda")]).astype(np.float64)
    y64 = oracle.gemv_w8a16_ref64(X16, q_o, s16_o, nthreads=oracle.num_threads())
    return W if rows is None else W[rows], X16, y, y64, q_o, s16_o


def test_chatglm2_w8a16_config():
    c = wl.CHATGLM2_W8A16
    say("chatglm2 W8A16", c["K"], c["N"])
    W, X16, y, y64, q8, s16 = _w8a16_case(c["seed"], wl.tensor_id("chatglm2", 0),
                                          wl.tensor_id("chatglm2", 1), 1, c["N"], c["K"])
    check_w8a16(y, X16, q8, s16, y64)
    yf = X16.astype(np.float64) @ W.astype(np.float64).T
    cos = float((y * yf).sum() / np.linalg.norm(y) / np.linalg.norm(yf))
    assert cos > 0.99


def test_headline_w8a16_shape():
    c = wl.HEADLINE
    say("headline W8A16", c["K"], c["N"])
    _, X16, y, y64, q8, s16 = _w8a16_case(7, wl.tensor_id("headline_w8", 0),
                                          wl.tensor_id("headline_w8", 1), 1, c["N"], c["K"])
    check_w8a16(y, X16, q8, s16, y64)


# ------------------------------------------------------------------ config 3 --

def _sample_rows(N, n=2048, seed=0):
    r = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(0, 64), np.arange(N - 64, N), r.choice(N, n, replace=False)])
    return np.unique(rows)


def test_lm_head_w4a8_full():
    """Every one of the 152064 rows: packed bytes, scales, int32 sums and outputs."""
    c = wl.LMHEAD_W4A8
    K, N = c["K"], c["N"]
    say("lm_head W4A8", K, N)
    W = wl.weights(c["seed"], wl.tensor_id("lm_head", 0), N, K)
    X = wl.activations(c["seed"], wl.tensor_id("lm_head", 1), 1, K)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    del W
    out = qw.gemv_w4a8_debug(dev(X), Wq, s)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert np.array_equal(host(out["Y"]).view(np.uint32), ref["Y"].view(np.uint32))
    Y = qw.gemv_w4a8(dev(X), Wq, s)
    assert np.array_equal(host(Y).view(np.uint32), ref["Y"].view(np.uint32))


# ------------------------------------------------------------------ config 4 --

@pytest.mark.parametrize("M", wl.SKINNY["Ms"])
def test_skinny_sweep_sampled(M):
    c = wl.SKINNY
    K, N = c["K"], c["N"]
    say("skinny", M, K, N)
    rows = _sample_rows(N, 512, seed=M)
    W = wl.weights(c["seed"], wl.tensor_id("skinny", 0), N, K)
    X = wl.activations(c["seed"], wl.tensor_id("skinny", 1), M, K)
    Wq, s, q_o, s_o = pack_w4_and_check(W, rows)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    ridx = torch.as_tensor(rows, device="cuda")
    Y = qw.gemv_w4a8(dev(X), Wq, s, workspace=qw.make_workspace("w4a8", M, N, K))
    assert_w4a8_close(host(Y[:, ridx]), ref["Y"])
    del Wq, s
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W, rows)
    y = qw.gemv_w8a16(dev(X16), Wq8, s16)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    check_w8a16(host(y[:, ridx]), X16, q8, s16_o, y64)


# ----------------------------------------------- skinny GEMM on the matrix cores --

# M >= 2 (W4A8) / M >= 3 (W8A16) runs the MFMA kernels: ragged M, N and K (K % 64 == 32
# leaves half a step)
MFMA_SHAPES = [(16, 64, 512), (17, 100, 544), (33, 257, 1056), (64, 128, 4096),
               (65, 70, 1024), (100, 300, 2080), (130, 36, 3584), (300, 200, 1568)]


@pytest.mark.parametrize("M,N,K", MFMA_SHAPES)
def test_skinny_gemm_full_parity(M, N, K):
    say("mfma", M, N, K)
    W = wl.weights(300 + M, 1, N, K, outlier_rows=N >= 100)
    W[0] = 0.0  # zero row
    X = wl.activations(300 + M, 2, M, K, outlier_channels=4)
    X[M // 2] = 0.0  # zero activation row
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    Xd = dev(X)
    Y = qw.gemv_w4a8(Xd, Wq, s, workspace=qw.make_workspace("w4a8", M, N, K))
    assert_w4a8_close(host(Y), ref["Y"])
    # the int32 sums are exact on both paths, so the GEMV kernels give the same bits
    Yg = qw.gemv_w4a8_tiled(Xd, Wq, s, 8, 4, 7)
    assert torch.equal(Y, Yg)
    assert not torch.any(Y[M // 2]).item() and not torch.any(Y[:, 0]).item()
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y = host(qw.gemv_w8a16(dev(X16), Wq8, s16))
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o)
    check_w8a16(y, X16, q8, s16_o, y64)
    assert not np.any(y[M // 2]) and not np.any(y[:, 0])


MFMA_LAUNCH = [(4, 1, 1), (4, 2, 1), (4, 4, 1), (4, 1, 2), (8, 1, 1), (8, 2, 2), (8, 4, 2),
               (4, 0, 1), (8, 0, 1)]


@pytest.mark.parametrize("M,N,K", [(1, 96, 512), (3, 70, 1056), (16, 257, 3584), (40, 300, 2080)])
def test_matrix_core_kernels_every_launch_shape(M, N, K):
    """The matrix-core kernels at small and ragged M (rows of X padded to 16), every
    launch shape: W4A8 equals the GEMV bit for bit, W8A16 is within the bar (its fp32
    sums start at a k that depends on the workgroup, so the last bits may differ
    between launch shapes)."""
    say("mfma shapes", M, N, K)
    W = wl.weights(500 + M, 1, N, K, outlier_rows=N >= 100)
    X = wl.activations(500 + M, 2, M, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    Xd = dev(X)
    Yg = qw.gemv_w4a8_tiled(Xd, Wq, s, 8, 4, 7)
    assert_w4a8_close(host(Yg), ref["Y"])
    X16 = X.astype(np.float16)
    X16d = dev(X16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o)
    for (nw, mb, nbw) in MFMA_LAUNCH:
        Y = qw.gemm_w4a8_mfma(Xd, Wq, s, nw, mb, nbw)
        assert torch.equal(Y, Yg), (nw, mb, nbw)
        if mb in (1, 2) and not (nw == 8 and nbw == 2):
            y = host(qw.gemm_w8a16_mfma(X16d, Wq8, s16, nw, mb, nbw))
            check_w8a16(y, X16, q8, s16_o, y64)


# The balanced matrix-core kernel (mb = 0): the ChatGLM2-shaped linear 4096 -> 27392 at
# 2 and 16 rows (its default range), ragged N (a partial row group and a partial block
# of 16 output rows), tiny N (fewer row groups than waves), 16 units per wave (N = 40000)
# and more workgroups than CUs (N = 70000, K = 4096), K not a multiple of 512
BALANCED_SHAPES = [(2, 27392, 4096), (4, 27392, 4096), (16, 27392, 4096), (5, 4101, 3584),
                   (16, 37, 96), (8, 37, 96), (3, 40000, 4096), (2, 70000, 4096),
                   (7, 1000, 1056), (1, 512, 4064), (6, 300, 544)]


@pytest.mark.parametrize("M,N,K", BALANCED_SHAPES)
def test_balanced_matrix_core_kernel_matches_oracle(M, N, K):
    say("balanced mfma", M, N, K)
    W = wl.weights(600 + M, 1, N, K, outlier_rows=True)
    X = wl.activations(600 + M, 2, M, K, outlier_channels=4)
    X[M // 2, : K // 3] = 0.0  # a partly zero row
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    ws = qw.make_workspace("w4a8", M, N, K)
    # the int32 sums are exact in any order: the streaming kernel gives the same bits
    Yg = host(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 1, 1, workspace=ws))
    assert_w4a8_close(Yg, ref["Y"])
    for nw in (8, 4):
        Y = host(qw.gemm_w4a8_mfma(Xd, Wq, s, nw, 0, 1, workspace=ws))
        assert np.array_equal(Y.view(np.uint32), Yg.view(np.uint32)), nw


# The balanced W4A8 kernel over 2 to 4 blocks of X (mb = 0, nbw = 2: weights held in
# registers across the blocks): 17 and 64 rows on 4096 -> 27392, ragged N and M, tiny N,
# K not a multiple of 512, more workgroups than CUs
BALANCED_MULTI_SHAPES = [(17, 27392, 4096), (64, 27392, 4096), (40, 4101, 3584), (33, 37, 96),
                         (50, 1000, 1056), (20, 70000, 4096), (63, 300, 544), (300, 4101, 3584),
                         (129, 2000, 1056), (1024, 260, 512)]


@pytest.mark.parametrize("M,N,K", BALANCED_MULTI_SHAPES)
def test_balanced_multi_block_kernel_matches_oracle(M, N, K):
    say("balanced multi-block mfma", M, N, K)
    W = wl.weights(800 + M, 1, N, K, outlier_rows=True)
    X = wl.activations(800 + M, 2, M, K, outlier_channels=4)
    X[M // 2] = 0.0  # a zero row
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    ws = qw.make_workspace("w4a8", M, N, K)
    Y = host(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 0, 2, workspace=ws))
    assert_w4a8_close(Y, ref["Y"])
    assert not np.any(Y[M // 2])
    # the int32 sums are exact in any order: the streaming kernel gives the same bits
    Yg = host(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 2, 1, workspace=ws))
    assert np.array_equal(Y.view(np.uint32), Yg.view(np.uint32))
    with pytest.raises(qw.QWError):
        qw.gemm_w4a8_mfma(Xd, Wq, s, 4, 0, 2, workspace=ws)


def test_balanced_multi_block_full_size_equals_streaming_kernel():
    """512 rows on 4096 -> 27392 (the sweep's largest M; the oracle would take minutes):
    the balanced kernel gives the streaming kernel's bits, and that kernel is held to the
    oracle at the other shapes."""
    M, N, K = 512, 27392, 4096
    say("balanced multi-block full size", M, N, K)
    W = wl.weights(900, 1, N, K, outlier_rows=True)
    X = wl.activations(900, 2, M, K, outlier_channels=4)
    Wq, s = qw.quantize_pack_w4(dev(W))
    Xd = dev(X)
    ws = qw.make_workspace("w4a8", M, N, K)
    Y = host(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 0, 2, workspace=ws))
    Yg = host(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 4, 1, workspace=ws))
    assert np.array_equal(Y.view(np.uint32), Yg.view(np.uint32))
    assert np.all(np.isfinite(Y)) and np.any(Y)
    with pytest.raises(qw.QWError):  # more than 1024 rows
        qw.gemm_w4a8_mfma(dev(wl.activations(901, 2, 1040, K)), Wq, s, 8, 0, 2,
                          workspace=qw.make_workspace("w4a8", 1040, N, K))


# The balanced W8A16 matrix-core kernel (mb = 0, one wave per 512-k step): the 4096 ->
# 27392 linear at 3 and 16 rows, ragged N, tiny N, one step (K = 512, more workgroups
# than CUs), K not a multiple of 512
W8_BALANCED_SHAPES = [(3, 27392, 4096), (16, 27392, 4096), (5, 4100, 3584), (16, 38, 96),
                      (7, 1000, 1056), (4, 40000, 512), (8, 600, 544)]


@pytest.mark.parametrize("M,N,K", W8_BALANCED_SHAPES)
def test_balanced_w8a16_matrix_core_kernel_matches_oracle(M, N, K):
    say("balanced w8a16 mfma", M, N, K)
    W = wl.weights(700 + M, 1, N, K, outlier_rows=True)
    X16 = wl.activations(700 + M, 2, M, K, outlier_channels=4).astype(np.float16)
    X16[M // 2, : K // 3] = 0
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    Xd = dev(X16)
    y = host(qw.gemm_w8a16_mfma(Xd, Wq8, s16, 8, 0, 1))
    check_w8a16(y, X16, q8, s16_o, y64)
    assert np.all(np.isfinite(y.astype(np.float32)))
    ys = host(qw.gemm_w8a16_mfma(Xd, Wq8, s16, 8, 1, 1))
    check_w8a16(ys, X16, q8, s16_o, y64)
    # the default path at these rows is the balanced kernel, unless there are enough
    # tiles of 128 x 32 for the tiled GEMM
    yd = host(qw.gemv_w8a16(Xd, Wq8, s16))
    if routed_to_tile(8, M, N):
        check_w8a16(yd, X16, q8, s16_o, y64)
    else:
        assert np.array_equal(yd.view(np.uint16), y.view(np.uint16))


W8_BALANCED_MULTI_SHAPES = [(17, 1000, 1056), (32, 27392, 4096), (40, 600, 544), (64, 4100, 3584),
                            (100, 38, 96), (300, 2050, 512), (33, 40000, 512)]


@pytest.mark.parametrize("M,N,K", W8_BALANCED_MULTI_SHAPES)
def test_balanced_w8a16_two_block_kernel_matches_oracle(M, N, K):
    """The balanced W8A16 kernel with two 16-row blocks of X per workgroup (nbw 2)."""
    say("balanced w8a16 mfma two blocks", M, N, K)
    W = wl.weights(720 + M, 1, N, K, outlier_rows=True)
    X16 = wl.activations(720 + M, 2, M, K, outlier_channels=4).astype(np.float16)
    X16[M // 2, : K // 3] = 0
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    Xd = dev(X16)
    y = host(qw.gemm_w8a16_mfma(Xd, Wq8, s16, 8, 0, 2))
    check_w8a16(y, X16, q8, s16_o, y64)
    assert np.all(np.isfinite(y.astype(np.float32)))
    # each row of X is summed in the same order as by the one-block kernel
    if M <= 16:
        y1 = host(qw.gemm_w8a16_mfma(Xd, Wq8, s16, 8, 0, 1))
        assert np.array_equal(y.view(np.uint16), y1.view(np.uint16))
    yd = host(qw.gemv_w8a16(Xd, Wq8, s16))
    check_w8a16(yd, X16, q8, s16_o, y64)
    # the default path at 17 to 64 rows is this kernel, except where the tiled GEMM
    # takes the rows
    tiled = routed_to_tile(8, M, N)
    if M <= 64 and not tiled:
        assert np.array_equal(yd.view(np.uint16), y.view(np.uint16))


def test_balanced_w8a16_kernel_limits():
    K, N = 512, 64
    W = wl.weights(730, 1, N, K)
    Wq8, s16, _, _ = pack_w8_and_check(W)
    X17 = dev(wl.activations(731, 2, 17, K).astype(np.float16))
    with pytest.raises(qw.QWError):
        qw.gemm_w8a16_mfma(X17, Wq8, s16, 8, 0, 1)  # one block: at most 16 rows
    X = dev(wl.activations(732, 2, 1025, K).astype(np.float16))
    with pytest.raises(qw.QWError):
        qw.gemm_w8a16_mfma(X, Wq8, s16, 8, 0, 2)  # two blocks: at most 1024 rows


def test_skinny_gemm_workspace_reuse_and_sizes():
    """One workspace sized for the larger call serves a smaller one after it."""
    K, N = 1024, 96
    W = wl.weights(400, 1, N, K)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ws = qw.make_workspace("w4a8", 80, N, K)
    for M in (80, 16, 48):
        X = wl.activations(400 + M, 2, M, K)
        ref = oracle.gemv_w4a8(X, q_o, s_o)
        Y = qw.gemv_w4a8(dev(X), Wq, s, workspace=ws)
        assert_w4a8_close(host(Y), ref["Y"])


# --------------------------------------------------------------- edge cases --

EDGE = [(1, 1, 32), (1, 5, 96), (2, 17, 64), (3, 517, 288), (5, 64, 1024), (8, 100, 3584),
        (9, 33, 256), (15, 7, 512), (1, 4100, 8192), (1, 3, 131072 // 8), (2, 37, 28672)]


@pytest.mark.parametrize("M,N,K", [(1, 37, 57344), (3, 5, 57344)])
def test_w4a8_at_its_largest_k(M, N, K):
    say("w4a8 max K", M, N, K)
    W = wl.weights(200 + M, 1, N, K, outlier_rows=False)
    X = wl.activations(200 + M, 2, M, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    out = qw.gemv_w4a8_debug(dev(X), Wq, s)
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert_w4a8_close(host(out["Y"]), ref["Y"])


@pytest.mark.parametrize("M,N,K", EDGE)
def test_edge_shapes_both_ops(M, N, K):
    say("edge", M, N, K)
    W = wl.weights(100 + M, 1, N, K, outlier_rows=N >= 100)
    if N > 2:
        W[1] = 0.0  # zero row
    X = wl.activations(100 + M, 2, M, K, outlier_channels=4 if K >= 64 else 0)
    if M > 1:
        X[M - 1] = 0.0  # zero activation vector
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    assert np.array_equal(host(qw.w4_codes(Wq, N, K)), q_o)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    out = qw.gemv_w4a8_debug(dev(X), Wq, s)
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert_w4a8_close(host(out["Y"]), ref["Y"])
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    assert np.array_equal(host(qw.w8_codes(Wq8, N, K)), q8)
    y = host(qw.gemv_w8a16(dev(X16), Wq8, s16))
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o)
    if np.linalg.norm(y64) > 0:
        check_w8a16(y, X16, q8, s16_o, y64)
    if M > 1:
        assert not np.any(y[M - 1]) and not np.any(host(out["Y"])[M - 1])


def launch_shapes(M, nrg4, nrg8, cg):
    """(u, nw, nwaves) combinations valid for both ops: u = 0 (register activations)
    only for M == 1, u = 1 (eager) with at most 16 tiles per wave, at most 64 row
    groups per wave."""
    out = []
    for u in ((0, 1, 2, 4, 8) if M == 1 else (1, 4, 8)):
        for nw in (4, 8, 16):
            for nwaves in (8, 13, 64, 100, 250, 333, 500, 1000):
                per4, per8 = -(-nrg4 // nwaves), -(-nrg8 // nwaves)
                if per4 > 64 or per8 > 64:
                    continue
                if u == 1 and max(per4, per8) * cg > 16:
                    continue
                if u == 2 and (nw != 4 or max(per4, per8) > 4):
                    continue  # all in flight: 4-wave workgroups, at most 4 row groups a wave
                out.append((u, nw, nwaves))
    return out


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_every_launch_shape_gives_the_same_result(M):
    K, N = 3584, 1000
    say("launch shapes M", M)
    W = wl.weights(55, 1, N, K, outlier_rows=True)
    X = wl.activations(55, 2, M, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o)
    Xd, X16d = dev(X), dev(X16)
    y_first = None
    shapes = launch_shapes(M, -(-N // 4), -(-N // 2), -(-K // 512))
    assert len(shapes) >= 12
    for (u, nw, nwaves) in shapes:
        Y = qw.gemv_w4a8_tiled(Xd, Wq, s, u, nw, nwaves)
        assert_w4a8_close(host(Y), ref["Y"])
        y = host(qw.gemv_w8a16_tiled(X16d, Wq8, s16, u, nw, nwaves))
        check_w8a16(y, X16, q8, s16_o, y64)
        # every launch shape adds a row's products in the same order
        if y_first is None:
            y_first = y
        assert np.array_equal(y.view(np.uint16), y_first.view(np.uint16)), (u, nw, nwaves)


# (N, K): at least 2048 row groups (the default path runs the producer variant), ragged
# N and K, one tile, one chunk, more workgroups than row groups
PRODUCER_SHAPES = [(8200, 3584), (9000, 4096), (4100, 1056), (2500, 2080), (333, 512), (37, 32)]


@pytest.mark.parametrize("N,K", PRODUCER_SHAPES)
def test_producer_wave_variant(N, K):
    """The producer-wave GEMV (u = 5) at every split of a workgroup into consumer and
    producer waves and at 1..301 workgroups gives the oracle's outputs; where the default
    path runs it (>= 2048 row groups), its debug outputs (int32 accumulators, activation
    codes and scale) equal the oracle's bit for bit."""
    say("producer variant N", N, "K", K)
    W = wl.weights(61, 1, N, K, outlier_rows=True)
    X = wl.activations(61, 2, 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    for (nw, P) in ((8, 2), (6, 2), (5, 3), (4, 4)):
        for blocks in (1, 3, 64, 256, 301):
            Y = qw.gemv_w4a8_tiled(Xd, Wq, s, 5, nw, blocks * nw, P)
            y = host(Y)
            assert_w4a8_close(y, ref["Y"])
            assert np.array_equal(y.view(np.uint32), ref["Y"].view(np.uint32)), (nw, P, blocks)
    if -(-N // 4) >= 2048:
        out = qw.gemv_w4a8_debug(Xd, Wq, s)
        assert np.array_equal(host(out["acc"]), ref["acc"])
        assert np.array_equal(host(out["xq"]), ref["xq"])
        assert np.array_equal(host(out["a"]).view(np.uint32), ref["a"].view(np.uint32))
        assert np.array_equal(host(out["Y"]).view(np.uint32), ref["Y"].view(np.uint32))
    with pytest.raises(qw.QWError):
        qw.gemv_w4a8_tiled(Xd, Wq, s, 5, 8, 8, 3)  # not a supported split
    with pytest.raises(qw.QWError):
        qw.gemv_w4a8_tiled(Xd, Wq, s, 5, 8, 12, 2)  # not whole workgroups


# (N, K) with K > 4096: the down projection, a short-N one, ragged K with 10, 16, 33 and
# 56 tiles per row (the largest K the split reaches, 7 tiles on each of 8 waves)
PRODUCER_SPLIT_SHAPES = [(3584, 18944), (512, 18944), (1000, 4640), (333, 8192), (4100, 16416),
                         (37, 28672)]


@pytest.mark.parametrize("N,K", PRODUCER_SPLIT_SHAPES)
def test_producer_wave_variant_split_k(N, K):
    """The producer-wave GEMV with K split over 2, 4 or 8 consumer waves (u = 6), at every
    valid split and several workgroup counts, gives the oracle's outputs bit for bit; the
    default path at M = 1 with K > 4096 runs it, debug outputs included."""
    say("producer variant split-K N", N, "K", K)
    W = wl.weights(62, 1, N, K, outlier_rows=True)
    X = wl.activations(62, 2, 1, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    nrg, cg = -(-N // 4), -(-K // 512)
    tried = 0
    for S in (2, 4, 8):
        if -(-cg // S) > 7:
            continue
        for blocks in sorted({-(-nrg // 16), 64, 256, 301}):
            if -(-nrg // blocks) > 16:
                continue
            y = host(qw.gemv_w4a8_tiled(Xd, Wq, s, 6, 8, blocks * 8, S))
            assert np.array_equal(y.view(np.uint32), ref["Y"].view(np.uint32)), (S, blocks)
            tried += 1
    assert tried >= 2
    out = qw.gemv_w4a8_debug(Xd, Wq, s)
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert np.array_equal(host(out["xq"]), ref["xq"])
    assert np.array_equal(host(out["a"]).view(np.uint32), ref["a"].view(np.uint32))
    y = host(qw.gemv_w4a8(Xd, Wq, s))
    assert np.array_equal(y.view(np.uint32), ref["Y"].view(np.uint32))
    with pytest.raises(qw.QWError):
        qw.gemv_w4a8_tiled(Xd, Wq, s, 6, 8, 8 * 256, 3)  # not a supported split


SPLITK_SHAPES = [(1, 512, 3584), (1, 100, 18944), (2, 37, 4640), (1, 4100, 1056), (2, 64, 32)]


@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
def test_split_k_launch_shapes(M, N, K):
    """Split-K inside the workgroup (2 or 4 waves per row run, each a k-slice) on ragged
    shapes, including slices that hold no tile: W4A8 equals the oracle to its bar and
    the unsplit launch bit for bit (int32 sums), W8A16 meets its bar."""
    say("split-K", M, N, K)
    W = wl.weights(600 + M, 1, N, K, outlier_rows=N >= 100)
    X = wl.activations(600 + M, 2, M, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o)
    Xd, X16d = dev(X), dev(X16)
    Y1 = qw.gemv_w4a8_tiled(Xd, Wq, s, 4, 4, max(1, -(-N // 4) // 2))
    assert_w4a8_close(host(Y1), ref["Y"])
    nrg4, nrg8 = -(-N // 4), -(-N // 2)
    n = n8 = 0
    for splitk in (2, 4):
        for u in (4, 8):
            for nw in (4, 8):
                for nwaves in (1, 3, 16, 100, 1000):
                    if -(-nrg4 // nwaves) > 16 or -(-nrg8 // nwaves) > 16 or nw < splitk:
                        continue
                    Y = qw.gemv_w4a8_tiled(Xd, Wq, s, u, nw, nwaves, splitk)
                    assert torch.equal(Y, Y1), (u, nw, nwaves, splitk)
                    n += 1
                    try:  # the f16 row of X, padded per k-slice, may not fit in LDS
                        y = host(qw.gemv_w8a16_tiled(X16d, Wq8, s16, u, nw, nwaves, splitk))
                    except qw.QWError as e:
                        assert e.status == qw.QW_ERR_TILING and K > 8192
                        continue
                    check_w8a16(y, X16, q8, s16_o, y64)
                    n8 += 1
    assert n >= 4 and n8 >= 2
    # all in flight with K in 8-tile slices (M == 1): 2..8 slices, 1..4 row groups a run
    if M == 1:
        cg = -(-K // 512)
        for S in sorted({max(2, -(-cg // 8)), max(2, -(-cg // 8)) + 1}):
            for per in (1, 2, 3, 4):
                y4 = qw.gemv_w4a8_tiled(Xd, Wq, s, 3, 4, -(-nrg4 // per), S)
                assert torch.equal(y4, Y1), ("flight split", S, per)
                if S <= 7:
                    y = host(qw.gemv_w8a16_tiled(X16d, Wq8, s16, 3, 4, -(-nrg8 // per), S))
                    check_w8a16(y, X16, q8, s16_o, y64)


# The balanced long-K W8A16 variant (u = 7): the 18944 -> 3584 down projection,
# K = 28672 (the longest W8A16 row), ragged N (a partial row group), tiny N (fewer row
# groups than workgroups), short K (one slice) and more than 8 row groups per workgroup;
# 2 to 9 rows of X (workgroups of 2 or 4 rows, a ragged last one)
W8_BSPLIT_SHAPES = [(1, 3584, 18944), (1, 512, 18944), (1, 301, 28672), (1, 5, 8192),
                    (1, 4100, 3584), (1, 640, 4608), (1, 2000, 96), (2, 3584, 18944),
                    (3, 512, 18944), (4, 301, 28672), (5, 2050, 8192), (9, 640, 4608),
                    (7, 38, 96)]


@pytest.mark.parametrize("M,N,K", W8_BSPLIT_SHAPES)
def test_balanced_long_k_w8a16_matches_oracle(M, N, K):
    say("w8a16 balanced long k", M, N, K)
    W = wl.weights(760 + N % 97, 1, N, K, outlier_rows=N >= 100)
    X16 = wl.activations(761 + N % 97, 2, M, K, outlier_channels=4).astype(np.float16)
    X16[M // 2, : K // 3] = 0
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    X16d = dev(X16)
    cg, nrg = -(-K // 512), -(-N // 2)
    ref = None
    n = 0
    s8 = max(1, -(-cg // 8))
    for S in sorted({s8, min(8, s8 + 1), 8, max(1, -(-cg // 4)), 16}):
        T = -(-cg // S)
        if T > 8 or S > (16 if T <= 4 and M == 1 else 8):
            continue
        for nwaves in sorted({1, 7, 256, -(-nrg // 16), nrg}):
            if nwaves > nrg or -(-nrg // nwaves) > 16:
                continue
            y = host(qw.gemv_w8a16_tiled(X16d, Wq8, s16, 7, S, nwaves, S))
            check_w8a16(y, X16, q8, s16_o, y64)
            assert np.all(np.isfinite(y.astype(np.float32)))
            # the slices' sums are added in slice order: the number of workgroups does
            # not change the bits
            if ref is None or ref[0] != S:
                ref = (S, y)
            else:
                assert np.array_equal(y.view(np.uint16), ref[1].view(np.uint16)), (S, nwaves)
            n += 1
    assert n >= 4
    yd = host(qw.gemv_w8a16(X16d, Wq8, s16))
    check_w8a16(yd, X16, q8, s16_o, y64)
    # the default path is this variant up to 8 rows (16 with weights below 24 MB)
    if cg > 8 and (M <= 8 or (M <= 16 and N * K < 24 << 20)) and (M >= 2 or nrg >= 1024):
        S = min(8, -(-cg // 4))
        yv = host(qw.gemv_w8a16_tiled(X16d, Wq8, s16, 7, S, -(-nrg // 16), S))
        assert np.array_equal(yd.view(np.uint16), yv.view(np.uint16))


def test_balanced_long_k_w8a16_limits():
    N, K = 64, 8192
    W = wl.weights(770, 1, N, K)
    Wq8, s16, _, _ = pack_w8_and_check(W)
    X16d = dev(wl.activations(771, 2, 1, K).astype(np.float16))
    for bad in [(7, 1, 2, 1),    # 16 tiles in one slice (at most 8)
                (7, 17, 2, 17),  # more than 16 waves
                (7, 4, 2, 2),    # nw must equal splitk (one wave per slice)
                (7, 2, 1, 2)]:   # 32 row groups on one workgroup (at most 16)
        with pytest.raises(qw.QWError):
            qw.gemv_w8a16_tiled(X16d, Wq8, s16, *bad)
    X2 = dev(wl.activations(772, 2, 2, K).astype(np.float16))
    qw.gemv_w8a16_tiled(X16d, Wq8, s16, 7, 16, 2, 16)  # 16 waves of one tile at M == 1 ...
    with pytest.raises(qw.QWError):
        qw.gemv_w8a16_tiled(X2, Wq8, s16, 7, 16, 2, 16)  # ... 8 at most from 2 rows
    N2, K2 = 64, 28672  # 56 tiles: 9 or 10 waves would take 7 or 6 tiles each (at most 8 waves)
    W2 = wl.weights(773, 1, N2, K2)
    Wq2, s2, _, _ = pack_w8_and_check(W2)
    X3 = dev(wl.activations(774, 2, 1, K2).astype(np.float16))
    for S in (9, 10):
        with pytest.raises(qw.QWError):
            qw.gemv_w8a16_tiled(X3, Wq2, s2, 7, S, 4, S)


# The balanced long-K W4A8 kernel: the 18944 -> 3584 down projection, short and ragged
# N, K = 32768 (the longest slice split, 8 tiles on each of 8 waves), short K; 1 to 16
# rows of X (workgroups of 1, 2 or 4 rows, a ragged last one)
W4_BSPLIT_SHAPES = [(1, 3584, 18944), (2, 3584, 18944), (3, 512, 18944), (4, 301, 32768),
                    (5, 2050, 8192), (9, 640, 4608), (16, 38, 96), (16, 1000, 18944),
                    (7, 6, 8192)]


@pytest.mark.parametrize("M,N,K", W4_BSPLIT_SHAPES)
def test_balanced_long_k_w4a8_matches_oracle(M, N, K):
    say("w4a8 balanced long k", M, N, K)
    W = wl.weights(780 + N % 97, 1, N, K, outlier_rows=N >= 100)
    X = wl.activations(781 + N % 97, 2, M, K, outlier_channels=4)
    X[M // 2, : K // 3] = 0
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    ws = torch.empty((qw.lib().qw_workspace_bytes(2, M, N, K),), dtype=torch.uint8, device="cuda")
    cg, nrg = -(-K // 512), -(-N // 4)
    s8 = max(1, -(-cg // 8))
    first = None
    n = 0
    for waves in sorted({s8, min(8, s8 + 1), 8, min(8, max(1, -(-cg // 4)))}):
        if -(-cg // waves) > 8:
            continue
        for wg in sorted({1, 7, 256, -(-nrg // 16), nrg}):
            if wg > nrg or -(-nrg // wg) > 16:
                continue
            Y = qw.gemv_w4a8_long_k(Xd, Wq, s, waves, wg, workspace=ws)
            if first is None:
                first = Y.clone()
                assert_w4a8_close(host(Y), ref["Y"])
            else:  # exact int32 sums: the same bits at every launch shape
                assert torch.equal(Y, first), (waves, wg)
            n += 1
    assert n >= 3
    Yd = qw.gemv_w4a8(Xd, Wq, s, workspace=ws)
    assert torch.equal(Yd, first)
    if M >= 2:
        assert torch.equal(qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 1, 1, workspace=ws), first)


@pytest.mark.parametrize("M,N,K", [(17, 600, 8192), (70, 300, 18944), (130, 520, 4608)])
def test_long_k_matrix_core_defaults_beyond_sixteen_rows(M, N, K):
    """K > 4096 from 17 rows: the default matrix-core shapes (4 waves up to 128 rows)
    give the oracle's W4A8 outputs and the same bits as another launch shape; W8A16
    within the bar."""
    say("long k mfma defaults", M, N, K)
    W = wl.weights(790 + M, 1, N, K, outlier_rows=True)
    X = wl.activations(791 + M, 2, M, K, outlier_channels=4)
    Wq, s, q_o, s_o = pack_w4_and_check(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    Xd = dev(X)
    ws = torch.empty((qw.lib().qw_workspace_bytes(2, M, N, K),), dtype=torch.uint8, device="cuda")
    Yd = qw.gemv_w4a8(Xd, Wq, s, workspace=ws)
    assert_w4a8_close(host(Yd), ref["Y"])
    assert torch.equal(Yd, qw.gemm_w4a8_mfma(Xd, Wq, s, 8, 2, 1, workspace=ws))
    X16 = X.astype(np.float16)
    Wq8, s16, q8, s16_o = pack_w8_and_check(W)
    y64 = oracle.gemv_w8a16_ref64(X16, q8, s16_o, nthreads=oracle.num_threads())
    y = host(qw.gemv_w8a16(dev(X16), Wq8, s16))
    check_w8a16(y, X16, q8, s16_o, y64)


def test_repeated_calls_are_deterministic():
    K, N, M = 4096, 2048, 1
    W = wl.weights(66, 1, N, K)
    X = wl.activations(66, 2, M, K)
    Wq, s = qw.quantize_pack_w4(dev(W))
    Wq8, s16 = qw.quantize_pack_w8(dev(W))
    ws4 = ws8 = None
    Xd, X16 = dev(X), dev(X.astype(np.float16))
    a = [host(qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)) for _ in range(3)]
    b = [host(qw.gemv_w8a16(X16, Wq8, s16, workspace=ws8)) for _ in range(3)]
    for i in (1, 2):
        assert np.array_equal(a[0].view(np.uint32), a[i].view(np.uint32))
        assert np.array_equal(b[0].view(np.uint16), b[i].view(np.uint16))


def test_packers_report_non_finite_weights():
    W = np.zeros((4, 64), np.float32)
    W[2, 5] = np.nan
    with pytest.raises(qw.QWError) as e:
        qw.quantize_pack_w4(dev(W))
    assert e.value.status == qw.QW_ERR_NONFINITE
    W[2, 5] = np.inf
    with pytest.raises(qw.QWError) as e:
        qw.quantize_pack_w8(dev(W))
    assert e.value.status == qw.QW_ERR_NONFINITE
    W[2, 5] = 1e7  # 1e7/127 overflows f16
    with pytest.raises(qw.QWError) as e:
        qw.quantize_pack_w8(dev(W))
    assert e.value.status == qw.QW_ERR_NONFINITE


def test_graph_capture_replays_match_eager():
    K, N, M = 3584, 512, 1
    W = wl.weights(77, 1, N, K)
    X = wl.activations(77, 2, M, K)
    Wq, s = qw.quantize_pack_w4(dev(W))
    Wq8, s16 = qw.quantize_pack_w8(dev(W))
    Xd, X16 = dev(X), dev(X.astype(np.float16))
    ws4 = ws8 = None
    e4 = host(qw.gemv_w4a8(Xd, Wq, s, workspace=ws4))
    e8 = host(qw.gemv_w8a16(X16, Wq8, s16, workspace=ws8))
    Y4 = torch.empty((M, N), device="cuda")
    Y8 = torch.empty((M, N), device="cuda", dtype=torch.float16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4, out=Y4)
        qw.gemv_w8a16(X16, Wq8, s16, workspace=ws8, out=Y8)
    for rep in range(4):
        Y4.fill_(float("nan"))
        Y8.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y4).view(np.uint32), e4.view(np.uint32)), rep
        assert np.array_equal(host(Y8).view(np.uint16), e8.view(np.uint16)), rep
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)  # eager work between replays


@pytest.mark.parametrize("M", [1, 2, 5, 12])
def test_long_k_graph_replays_match_eager(M):
    """The long-K defaults (the producer-wave W4A8 GEMV and the balanced long-K W8A16
    variant at one row; the balanced long-K kernels, with the W4A8 row quantization
    into the workspace, from two) captured in one graph: every replay, with eager work
    between replays, gives the eager bits."""
    K, N = 8192, 1000
    say("long-k graph replays M", M)
    W = wl.weights(1300 + M, 1, N, K)
    X = wl.activations(1300 + M, 2, M, K)
    Wq, s = qw.quantize_pack_w4(dev(W))
    Wq8, s16 = qw.quantize_pack_w8(dev(W))
    Xd, X16 = dev(X), dev(X.astype(np.float16))
    ws4 = qw.make_workspace("w4a8", M, N, K)
    e4 = host(qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)).copy()
    e8 = host(qw.gemv_w8a16(X16, Wq8, s16)).copy()
    Y4 = torch.empty((M, N), device="cuda")
    Y8 = torch.empty((M, N), device="cuda", dtype=torch.float16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4, out=Y4)
        qw.gemv_w8a16(X16, Wq8, s16, out=Y8)
    for rep in range(4):
        Y4.fill_(float("nan"))
        Y8.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y4).view(np.uint32), e4.view(np.uint32)), rep
        assert np.array_equal(host(Y8).view(np.uint16), e8.view(np.uint16)), rep
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)  # eager work between replays
        qw.gemv_w8a16(X16, Wq8, s16)


@pytest.mark.parametrize("M", [4, 20, 40, 64])
def test_matrix_core_graph_replays_match_eager(M):
    """The matrix-core defaults (balanced kernels up to 16 rows; the W4A8 kernel over many
    blocks of X, unpaired at 20 rows and paired from 40; W8A16 streaming past 16 rows)
    captured in one graph: every replay, with eager work between replays, gives the
    eager bits (both variants are deterministic)."""
    K, N = 1056, 1000
    say("matrix-core graph replays M", M)
    W = wl.weights(1200 + M, 1, N, K)
    X = wl.activations(1200 + M, 2, M, K)
    Wq, s = qw.quantize_pack_w4(dev(W))
    Wq8, s16 = qw.quantize_pack_w8(dev(W))
    Xd, X16 = dev(X), dev(X.astype(np.float16))
    ws4 = qw.make_workspace("w4a8", M, N, K)
    e4 = host(qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)).copy()
    e8 = host(qw.gemv_w8a16(X16, Wq8, s16)).copy()
    Y4 = torch.empty((M, N), device="cuda")
    Y8 = torch.empty((M, N), device="cuda", dtype=torch.float16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4, out=Y4)
        qw.gemv_w8a16(X16, Wq8, s16, out=Y8)
    for rep in range(4):
        Y4.fill_(float("nan"))
        Y8.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y4).view(np.uint32), e4.view(np.uint32)), rep
        assert np.array_equal(host(Y8).view(np.uint16), e8.view(np.uint16)), rep
        qw.gemv_w4a8(Xd, Wq, s, workspace=ws4)  # eager work between replays
        qw.gemv_w8a16(X16, Wq8, s16)

