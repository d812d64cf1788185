"""Rounding edge cases of every quantizer on the GPU, against the CPU oracle.

The method's codes are q = clamp(rint(v / s), -qmax, qmax) with s = maxabs / qmax
("Jetson Orin AGX 上的 INT4 量化推理实践", section 当前实现方式, for INT4 weights and
the dynamic INT8 activations; the ChatGLM2-6B W8A16 write-up, sections 2 and 3, for
INT8 weights with an f16 scale) and rint rounds half to even.  The inputs here sit on
and around the rounding boundaries:

* tie rows: entries at (c + 1/2) * s with s a power of two, so v / s is exactly a
  half-integer and only round-half-to-even decides (2.5 -> 2, 3.5 -> 4, -2.5 -> -2);
* closed-form rows: entries c * 2^-e with a +-qmax present, whose scale is exactly
  2^-e and whose codes are exactly c;
* near-tie rows: entries a few ulps either side of (c + 1/2) * s for scales that are
  not powers of two.  The GPU activation quantizers multiply by 1 / s and fall back
  to the division only when the product lies within 2^-15 of a half-integer; these
  rows put values on both sides of that window;
* W8 rows whose f16 scale underflows to zero (a zero row), and whose f16 scale rounds
  down so that the largest entry divides to more than 127.5 and clamps.

Each quantizer is checked where its codes can be read: the packers through the code
decoders, the standalone quantizer directly, the GEMV prologues through the debug
outputs, the matrix-core pre-pass and the long-K row pre-pass through their
workspaces (decoded here from the documented layouts).  Codes and scales must equal
the oracle's bit for bit, and the outputs computed from them too.
"""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import oracle

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


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


# ------------------------------------------------------------ input builders --

def tie_row(K, qmax, e, rng):
    """(c + 1/2) * 2^-e for c across the code range, a +qmax entry first (scale 2^-e),
    padded with closed-form entries c * 2^-e; shuffled except the first entry."""
    half = np.arange(-qmax, qmax, dtype=np.float64) + 0.5
    vals = np.concatenate([half, rng.integers(-qmax, qmax + 1, size=max(0, K - 1 - half.size))])
    vals = vals[:K - 1]
    rng.shuffle(vals)
    return (np.concatenate([[qmax], vals]) * 2.0 ** -e).astype(np.float32)


def near_tie_row(K, qmax, scale_of, m, rng, ulps=(0, 1, 2, 3, 5, 8, 64, 512, 2048)):
    """Entries a few ulps either side of fl((c + 1/2) * s), s the scale the quantizer
    derives from maxabs m (which is the first entry), c across the code range."""
    s = np.float64(scale_of(np.float32(m)))
    out = [np.float32(m)]
    cs = np.arange(-qmax, qmax, dtype=np.float64) + 0.5
    while len(out) < K:
        c = cs[rng.integers(0, cs.size)]
        d = int(ulps[rng.integers(0, len(ulps))]) * int(rng.choice([-1, 1]))
        x = np.float32(c * s)
        x = (x.view(np.int32) + np.int32(d)).view(np.float32) if x != 0 else x
        if abs(float(x)) <= float(m):
            out.append(np.float32(x))
    return np.array(out, np.float32)


def act_scale(m):
    return np.float32(m) / np.float32(127)


def w4_scale(m):
    return np.float32(m) / np.float32(7)


def w8_scale(m):
    return np.float32(np.float32(m) / np.float32(127)).astype(np.float16).astype(np.float32)


def edge_matrix(R, K, qmax, scale_of, seed):
    """R rows: ties at 2^-3 and 2^-9, a closed-form row, then near-tie rows at scales
    that are not powers of two (one with a subnormal-range reciprocal-free scale)."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(R):
        kind = i % 6
        if kind == 0:
            rows.append(tie_row(K, qmax, 3, rng))
        elif kind == 1:
            rows.append(tie_row(K, qmax, 9, rng))
        elif kind == 2:
            c = rng.integers(-qmax, qmax + 1, size=K).astype(np.float64)
            c[rng.integers(0, K)] = -qmax
            rows.append((c * 2.0 ** -5).astype(np.float32))
        else:
            m = [3.7, 20.123, 0.0123457, 1.0e-3 * np.pi][(i // 6 + kind) % 4]
            r = near_tie_row(K, qmax, scale_of, m, rng)
            rng.shuffle(r[1:])
            rows.append(r)
    return np.stack(rows)


# ---------------------------------------------------------- workspace layouts --

def mfma_ws_codes(ws, M, K):
    """The matrix-core pre-pass workspace -> (codes int8 [M][K], scales fp32 [M]).
    Layout: rows of X in blocks of 16, 64-k steps; block b, step st, lane group g
    (16 k) hold 16 bytes per row r = m % 16 at ((b * KS + st) * 1024 + g * 256 + r * 16);
    inside, bytes 0-3 hold k = 16g + 0, 2, 4, 6; bytes 4-7 k + 1, 3, 5, 7; bytes 8-11
    k + 8, 10, 12, 14; bytes 12-15 k + 9, 11, 13, 15.  The scales follow the codes at
    the next multiple of 256 bytes."""
    ws = host(ws).view(np.uint8)
    KS = -(-K // 64)
    mbt = -(-M // 16)
    xp = (mbt * KS * 1024 + 255) // 256 * 256
    order = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]  # k offset of byte i
    codes = np.zeros((M, KS * 64), np.int8)
    blk = ws[:mbt * KS * 1024].reshape(mbt, KS, 4, 16, 16)  # [b][st][g][r][byte]
    for m in range(M):
        b, r = divmod(m, 16)
        v = blk[b, :, :, r, :].view(np.int8)  # [st][g][byte]
        for i, off in enumerate(order):
            codes[m, (np.arange(KS)[:, None] * 64 + np.arange(4)[None, :] * 16 + off).ravel()] = \
                v[:, :, i].ravel()
    a = ws[xp:xp + 4 * M].view(np.float32)
    return codes[:, :K], a


def rows_ws_codes(ws, M, K):
    """The long-K row pre-pass workspace -> (codes int8 [M][K] row-major, scales [M]);
    the scales follow the codes at the next multiple of 256 bytes."""
    ws = host(ws).view(np.uint8)
    off = (M * K + 255) // 256 * 256
    return ws[:M * K].view(np.int8).reshape(M, K), ws[off:off + 4 * M].view(np.float32)


# ------------------------------------------------------------------- packers --

@pytest.mark.parametrize("N,K", [(36, 512), (13, 1056), (24, 3584)])
def test_pack_w4_ties_and_near_ties(N, K):
    say("pack_w4 edges", N, K)
    W = edge_matrix(N, K, 7, w4_scale, 10 + N)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    assert np.array_equal(bits(host(s)), bits(s_o))
    assert np.array_equal(host(qw.w4_codes(Wq, N, K)), q_o)
    # the half-to-even decisions of the tie rows, from the page's formula alone
    for i in (0, 1):
        e = 3 if i == 0 else 9
        t = W[i].astype(np.float64) * 2.0 ** e
        tie = np.abs(t - np.round(t)) == 0.5
        assert tie.sum() >= 14
        assert np.all(q_o[i][tie] % 2 == 0)


@pytest.mark.parametrize("group", [32, 128])
def test_pack_w4g_ties_and_near_ties(group):
    N, K = 12, 1024
    say("pack_w4g edges", group)
    W = edge_matrix(N, K, 7, w4_scale, 20 + group)
    Wq, s = qw.quantize_pack_w4g(dev(W), group)
    q_o, s_o = oracle.quant_w4g(W, group)
    assert np.array_equal(host(qw.w4_codes(Wq, N, K)), q_o)
    assert np.array_equal(bits(host(qw.w4g_scales(s, N, K, group))), bits(s_o))


@pytest.mark.parametrize("N,K", [(30, 512), (7, 2080), (12, 4096)])
def test_pack_w8_ties_and_near_ties(N, K):
    say("pack_w8 edges", N, K)
    W = edge_matrix(N, K, 127, w8_scale, 30 + N)
    Wq, s16 = qw.quantize_pack_w8(dev(W))
    q_o, s16_o = oracle.quant_w8(W)
    assert np.array_equal(bits(host(s16)), s16_o)
    assert np.array_equal(host(qw.w8_codes(Wq, N, K)), q_o)


def test_pack_w8_scale_underflow_and_clamp_rows():
    """Row 0: maxabs / 127 below half the smallest f16 subnormal, so the stored scale is
    0 and the row is a zero row.  Row 1: a maxabs whose f16 scale rounds down in the
    subnormal range, so the largest entry divides to more than 127.5 and clamps to 127.
    Row 2: the same with the sign flipped (clamps to -127).  Row 3: an ordinary row."""
    K = 64
    cand = np.float32(1e-4) + np.arange(4000, dtype=np.float32) * np.float32(1e-7)
    s16f = (cand / np.float32(127)).astype(np.float16).astype(np.float32)
    m = cand[(cand / s16f) > np.float32(127.5)][0]
    W = np.zeros((4, K), np.float32)
    W[0, :5] = [2.0e-6, -1.5e-6, 1.0e-6, 0.5e-6, -2.0e-6]  # 2e-6 / 127 < 2^-25
    W[1, :4] = [m, -m / 2, m / 3, m / 5]
    W[2, :4] = [-m, m / 2, -m / 3, m / 7]
    W[3] = np.linspace(-1.0, 0.75, K, dtype=np.float32)
    Wq, s16 = qw.quantize_pack_w8(dev(W))
    q_o, s16_o = oracle.quant_w8(W)
    sh = bits(host(s16))
    assert np.array_equal(sh, s16_o)
    codes = host(qw.w8_codes(Wq, 4, K))
    assert np.array_equal(codes, q_o)
    assert sh[0] == 0 and not codes[0].any()
    assert codes[1, 0] == 127 and codes[2, 0] == -127
    # the zero-scale row gives exact zeros downstream
    X16 = np.ones((1, K), np.float16)
    y = host(qw.gemv_w8a16(dev(X16), Wq, s16))
    assert y[0, 0] == 0


# ------------------------------------------------------ activation quantizers --

def _act_edges(M, K, seed):
    X = edge_matrix(M, K, 127, act_scale, seed)
    if M >= 4:
        X[3] = 0.0  # an all-zero vector: scale 0, codes 0
    return X


@pytest.mark.parametrize("M,K", [(6, 256), (7, 3584), (3, 18944), (12, 1056)])
def test_quant_act_i8_ties_and_near_ties(M, K):
    say("quant_act_i8 edges", M, K)
    X = _act_edges(M, K, 40 + K)
    xq, a = qw.quant_act_i8(dev(X))
    xq_o, a_o = oracle.quant_act_i8(X)
    assert np.array_equal(bits(host(a)), bits(a_o))
    assert np.array_equal(host(xq), xq_o)
    # ties resolve to even codes
    t = X[0].astype(np.float64) * 2.0 ** 3
    tie = np.abs(t - np.round(t)) == 0.5
    assert tie.sum() >= 200 and np.all(xq_o[0][tie] % 2 == 0)


# M == 1 rows on the producer-wave GEMV: K <= 4096 (one k-slice per consumer, from 2048
# row groups 8 + 2 waves, below 4 + 4) and K > 4096 (K split over consumer waves)
@pytest.mark.parametrize("row,N,K", [(0, 8200, 3584), (1, 512, 3584), (3, 64, 2080),
                                     (4, 3584, 18944), (5, 100, 8192), (0, 40, 28672)])
def test_fused_prologue_ties_and_near_ties(row, N, K):
    say("fused prologue edges", row, N, K)
    X = _act_edges(6, K, 50 + K)[row:row + 1]
    rng = np.random.default_rng(N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    out = qw.gemv_w4a8_debug(dev(X), Wq, s)
    assert np.array_equal(host(out["xq"]), ref["xq"])
    assert np.array_equal(bits(host(out["a"])), bits(ref["a"]))
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert np.array_equal(bits(host(out["Y"])), bits(ref["Y"]))


@pytest.mark.parametrize("M,K", [(2, 512), (20, 3584), (17, 8192), (5, 16384), (3, 18944),
                                 (2, 57344)])
def test_matrix_core_prepass_ties_and_near_ties(M, K):
    """k_quant_act_mfma at every width it is built for (one to four 16-code slots per
    thread of 256, two to four per thread of 1024)."""
    say("matrix-core pre-pass edges", M, K)
    X = _act_edges(M, K, 60 + K)
    N = 40
    rng = np.random.default_rng(K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    ws = qw.make_workspace("w4a8", M, N, K)
    ws.fill_(0x55)
    Y = qw.gemm_w4a8_mfma(dev(X), Wq, s, 8, 1, 1, workspace=ws)
    codes, a = mfma_ws_codes(ws, M, K)
    assert np.array_equal(bits(a), bits(ref["a"]))
    assert np.array_equal(codes, ref["xq"])
    assert np.array_equal(bits(host(Y)), bits(ref["Y"]))


@pytest.mark.parametrize("M,K", [(2, 8192), (4, 18944), (3, 4608)])
def test_long_k_row_prepass_ties_and_near_ties(M, K):
    say("long-K row pre-pass edges", M, K)
    X = _act_edges(6, K, 70 + K)[:M]
    N = 36
    rng = np.random.default_rng(K + 1)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    ws = torch.full((qw.lib().qw_workspace_bytes(2, M, N, K),), 0x55, dtype=torch.uint8,
                    device="cuda")
    cg = -(-K // 512)
    Y = qw.gemv_w4a8_long_k(dev(X), Wq, s, min(8, -(-cg // 4)), 3, workspace=ws)
    codes, a = rows_ws_codes(ws, M, K)
    assert np.array_equal(bits(a), bits(ref["a"]))
    assert np.array_equal(codes, ref["xq"])
    assert np.array_equal(bits(host(Y)), bits(ref["Y"]))


@pytest.mark.parametrize("M,K", [(2, 4096), (3, 3584), (4, 1056), (4, 4096), (1, 512)])
def test_balanced_fused_prologue_ties_and_near_ties(M, K):
    """Up to 4 rows, the balanced matrix-core kernel quantizes X in its own prologue
    (no pre-pass launch): with tie and near-tie activations, and an all-zero row at 4
    rows, its outputs (exact int32 sums, fixed epilogue) equal the oracle's bit for bit
    on the default path and at an explicit launch shape."""
    say("balanced fused prologue edges", M, K)
    X = _act_edges(max(M, 6), K, 100 + K)[:M]
    N = 300
    rng = np.random.default_rng(K + 3)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    ws = qw.make_workspace("w4a8", M, N, K)
    if M >= 2:
        Y = qw.gemv_w4a8(dev(X), Wq, s, workspace=ws)
        assert np.array_equal(bits(host(Y)), bits(ref["Y"]))
    Y8 = qw.gemm_w4a8_mfma(dev(X), Wq, s, 8, 0, 1,
                           workspace=ws if ws is not None else qw.make_workspace("w4a8", 2, N, K))
    assert np.array_equal(bits(host(Y8)), bits(ref["Y"]))


UNPACK_ORDER = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]  # k offset of byte i


@pytest.mark.parametrize("variant", [0, 4])
@pytest.mark.parametrize("M,K", [(5, 4096), (3, 18944), (2, 512)])
def test_tiled_gemm_prepass_ties_and_near_ties(variant, M, K):
    """The row pre-pass of the tiled GEMM: row-major codes, each 16-byte group holding
    its 16 k in the INT4 unpack order (byte i of group g = k 16 g + UNPACK_ORDER[i])."""
    say("tiled GEMM pre-pass edges", variant, M, K)
    X = _act_edges(6, K, 90 + K)[:M]
    N = 40
    rng = np.random.default_rng(K + 2)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o, nthreads=oracle.num_threads())
    ws = torch.full((qw.lib().qw_workspace_bytes(2, M, N, K),), 0x55, dtype=torch.uint8,
                    device="cuda")
    Y = qw.gemm_w4a8_tile(dev(X), Wq, s, variant, workspace=ws)
    codes, a = rows_ws_codes(ws, M, K)
    codes = codes.reshape(M, K // 16, 16)[:, :, np.argsort(UNPACK_ORDER)].reshape(M, K)
    assert np.array_equal(bits(a), bits(ref["a"]))
    assert np.array_equal(codes, ref["xq"])
    assert np.array_equal(bits(host(Y)), bits(ref["Y"]))


@pytest.mark.parametrize("M,u", [(1, 0), (1, 2), (1, 4), (2, 1), (3, 8)])
def test_gemv_variant_prologues_ties_and_near_ties(M, u):
    """The register, all-in-flight, eager and streaming GEMV variants quantize X in
    their own prologue; with tie and near-tie activations their outputs (exact int32
    sums, fixed epilogue) equal the oracle's bit for bit."""
    K, N = 3584, 300
    say("GEMV variant prologue edges", M, u)
    X = _act_edges(6, K, 80 + u)[:M]
    rng = np.random.default_rng(u)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wq, s = qw.quantize_pack_w4(dev(W))
    q_o, s_o = oracle.quant_w4(W)
    ref = oracle.gemv_w4a8(X, q_o, s_o)
    nrg = -(-N // 4)
    Y = qw.gemv_w4a8_tiled(dev(X), Wq, s, u, 4, nrg if u != 1 else nrg)
    assert np.array_equal(bits(host(Y)), bits(ref["Y"]))
