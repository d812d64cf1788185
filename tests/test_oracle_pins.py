"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something fixed by the pages or by mathematics:
closed-form inputs whose codes are known in advance, rounding ties, invariants of
symmetric quantization, exact rational arithmetic, brute force on tiny inputs, an
independent binary16 implementation (numpy's), and the storage figures printed in
the ChatGLM2-6B W8A16 write-up.  A dropped term, a flipped sign, a swapped nibble or
a transposed operand in the oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- binary16 --

def test_f32_from_f16_exhaustive_against_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f32_from_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_round_trip_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f32_from_f16(h)
    back = oracle.f16_from_f32(f)
    finite = (h & 0x7C00) != 0x7C00
    inf = ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) == 0)
    assert np.array_equal(back[finite | inf], h[finite | inf])
    nan = ~(finite | inf)
    assert np.all((back[nan] & 0x7C00) == 0x7C00) and np.all((back[nan] & 0x3FF) != 0)


def test_f16_from_f32_matches_numpy_rne():
    rng = np.random.default_rng(123)
    parts = [
        rng.standard_normal(1_000_000).astype(np.float32),
        (rng.standard_normal(500_000) * 1e-5).astype(np.float32),       # subnormal halves
        (rng.standard_normal(200_000) * 3e4).astype(np.float32),        # near overflow
        rng.integers(0, 2**32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    # every binary16 midpoint (exactly between two neighbours): ties go to even
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    parts.append(np.array([65504, 65519.996, 65520, 65536, 1e-8, 2.98e-8, 2.99e-8, -0.0, 0.0],
                          np.float32))
    x = np.concatenate(parts)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_from_f32(x), ref)


# ------------------------------------------------------------ INT4 weights --

def _pow2_rows(rng, N, K, qmax, e):
    """Rows W = c * 2^-e with integer c in [-qmax, qmax] and one entry at +-qmax."""
    c = rng.integers(-qmax, qmax + 1, size=(N, K))
    pos = rng.integers(0, K, size=N)
    sgn = rng.choice([-1, 1], size=N)
    c[np.arange(N), pos] = sgn * qmax
    return (c * 2.0 ** -e).astype(np.float32), c


def test_quant_w4_closed_form_rows():
    rng = np.random.default_rng(1)
    for e in (0, 3, 7, 12):
        W, c = _pow2_rows(rng, 9, 40, 7, e)
        q, s = oracle.quant_w4(W)
        assert np.all(s == np.float32(2.0 ** -e))
        assert np.array_equal(q, c)


def test_quant_w4_ties_round_half_to_even():
    s = 2.0 ** -5
    row = np.array([7, -7, 2.5, -2.5, 3.5, -3.5, 0.5, -0.5, 1.5, -1.5, 4.5, 5.5, 6.5, -6.5], np.float64)
    W = (row * s).astype(np.float32)[None, :]
    q, sc = oracle.quant_w4(W)
    assert sc[0] == np.float32(s)
    assert q[0].tolist() == [7, -7, 2, -2, 4, -4, 0, 0, 2, -2, 4, 6, 6, -6]


def test_quant_w4_zero_row_and_invariants():
    W = workloads.weights(11, 1, 64, 96, outlier_rows=True)
    W[5] = 0.0
    q, s = oracle.quant_w4(W)
    assert s[5] == 0 and not q[5].any()
    nz = np.arange(64) != 5
    assert np.abs(q).max() <= 7
    assert np.all(np.abs(q[nz]).max(axis=1) == 7)
    # s = maxabs / 7 in fp32, bit for bit
    assert np.array_equal(s, np.abs(W).max(axis=1) / np.float32(7))
    # reconstruction: |W - q s| <= s/2 up to one fp32 rounding of W/s
    err = np.abs(W.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -20))


def test_quant_w4_symmetries():
    W = workloads.weights(12, 1, 32, 64)
    q, s = oracle.quant_w4(W)
    qn, sn = oracle.quant_w4(-W)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    q2, s2 = oracle.quant_w4(W * np.float32(2.0 ** 9))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** 9))
    perm = np.random.default_rng(3).permutation(64)
    qp, sp = oracle.quant_w4(W[:, perm])
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(sp, s)


def test_quant_w4_rejects_non_finite():
    W = np.zeros((2, 8), np.float32)
    W[1, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quant_w4(W)


def test_pack_w4_hand_computed_bytes():
    q = np.array([[-1, 3, 7, -7, 0, -8, 1, 0]], np.int8)
    p = oracle.pack_w4(q)
    # low nibble = even k, two's complement: (-1, 3) -> 0x3F, (7, -7) -> 0x97,
    # (0, -8) -> 0x80, (1, 0) -> 0x01
    assert p[0].tolist() == [0x3F, 0x97, 0x80, 0x01]


def test_pack_unpack_exhaustive_pairs():
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], axis=1).reshape(1, -1).astype(np.int8)
    p = oracle.pack_w4(q)
    assert sorted(p[0].tolist()) == list(range(256))  # a bijection on bytes
    assert np.array_equal(oracle.unpack_w4(p, q.shape[1]), q)


# ------------------------------------------------------- INT8 activations --

def test_quant_act_closed_form_and_ties():
    rng = np.random.default_rng(5)
    X, c = _pow2_rows(rng, 3, 77, 127, 4)
    xq, a = oracle.quant_act_i8(X)
    assert np.all(a == np.float32(2.0 ** -4)) and np.array_equal(xq, c)
    s = 2.0 ** -2
    row = np.array([127, 0.5, 1.5, 2.5, -2.5, 100.5, 101.5, -126.5, 126.5], np.float64)
    xq, a = oracle.quant_act_i8((row * s).astype(np.float32)[None, :])
    assert xq[0].tolist() == [127, 0, 2, 2, -2, 100, 102, -126, 126]


def test_quant_act_invariants():
    X = workloads.activations(7, 2, 4, 3584, outlier_channels=4)
    xq, a = oracle.quant_act_i8(X)
    assert np.array_equal(a, np.abs(X).max(axis=1) / np.float32(127))
    assert np.all(np.abs(xq).max(axis=1) == 127) and np.abs(xq).max() <= 127
    err = np.abs(X.astype(np.float64) - xq * a[:, None].astype(np.float64))
    assert np.all(err <= a[:, None] * (0.5 + 2.0 ** -16))
    z, az = oracle.quant_act_i8(np.zeros((1, 64), np.float32))
    assert az[0] == 0 and not z.any()


# ------------------------------------------------------------- W4A8 linear --

def _brute_acc(q, xq):
    M, K = xq.shape
    N = q.shape[0]
    return [[sum(int(q[n, k]) * int(xq[m, k]) for k in range(K)) for n in range(N)] for m in range(M)]


def test_gemv_w4a8_brute_force_and_exact_identity():
    W = workloads.weights(21, 1, 6, 24)
    X = workloads.activations(21, 2, 3, 24)
    q, s = oracle.quant_w4(W)
    r = oracle.gemv_w4a8(X, q, s)
    assert r["acc"].tolist() == _brute_acc(q, r["xq"])
    for m in range(3):
        for n in range(6):
            # exact rationals: sum_k (q s)(xq a) == acc * s * a
            exact = sum(Fraction(int(q[n, k])) * Fraction(float(s[n])) * Fraction(int(r["xq"][m, k]))
                        * Fraction(float(r["a"][m])) for k in range(24))
            assert exact == Fraction(int(r["acc"][m, n])) * Fraction(float(s[n])) * Fraction(float(r["a"][m]))
            # Y is that value after two fp32 roundings (acc*s, then *a)
            y = Fraction(float(r["Y"][m, n]))
            if exact != 0:
                assert abs(y - exact) / abs(exact) <= Fraction(1, 2 ** 22)
            else:
                assert y == 0


def test_gemv_w4a8_against_fp64_dequantized_matmul():
    W = workloads.weights(22, 1, 300, 512, outlier_rows=True)
    X = workloads.activations(22, 2, 2, 512, outlier_channels=4)
    q, s = oracle.quant_w4(W)
    r = oracle.gemv_w4a8(X, q, s)
    y64 = (r["xq"].astype(np.float64) * r["a"][:, None]) @ (q.astype(np.float64) * s[:, None]).T
    rel = np.abs(r["Y"] - y64) / np.maximum(np.abs(y64), 1e-30)
    assert np.all(rel[y64 != 0] <= 2.0 ** -22)
    assert np.all(r["Y"][y64 == 0] == 0)
    # the integer accumulator equals the int64 matmul of the codes
    assert np.array_equal(r["acc"], r["xq"].astype(np.int64) @ q.astype(np.int64).T)


def test_gemv_w4a8_one_hot_picks_a_column():
    W = workloads.weights(23, 1, 40, 64)
    q, s = oracle.quant_w4(W)
    X = np.zeros((1, 64), np.float32)
    X[0, 13] = -0.75
    r = oracle.gemv_w4a8(X, q, s)
    assert r["xq"][0, 13] == -127 and r["a"][0] == np.float32(0.75) / np.float32(127)
    assert np.array_equal(r["acc"][0], -127 * q[:, 13].astype(np.int32))


def test_gemv_w4a8_symmetries_and_threads():
    W = workloads.weights(24, 1, 128, 256)
    X = workloads.activations(24, 2, 3, 256)
    q, s = oracle.quant_w4(W)
    r = oracle.gemv_w4a8(X, q, s)
    rn = oracle.gemv_w4a8(-X, q, s)
    assert np.array_equal(rn["Y"], -r["Y"])
    r2 = oracle.gemv_w4a8(X * np.float32(2.0 ** -6), q, s)
    assert np.array_equal(r2["Y"], r["Y"] * np.float32(2.0 ** -6))
    perm = np.random.default_rng(9).permutation(256)
    rp = oracle.gemv_w4a8(X[:, perm], q[:, perm], s)
    assert np.array_equal(rp["Y"], r["Y"])
    rt = oracle.gemv_w4a8(X, q, s, nthreads=4)
    assert np.array_equal(rt["Y"], r["Y"]) and np.array_equal(rt["acc"], r["acc"])


# --------------------------------------------------- group-wise INT4 scales --

def test_quant_w4g_closed_form_groups():
    """Each group c * 2^-e_t with a +-7 present: its scale is exactly 2^-e_t and its codes
    are c, whatever the other groups of the row hold."""
    rng = np.random.default_rng(41)
    N, g, G = 7, 64, 5
    es = [0, 3, 9, 1, 12]
    W = np.empty((N, g * G), np.float32)
    C = np.empty((N, g * G), np.int8)
    for t, e in enumerate(es):
        Wt, ct = _pow2_rows(rng, N, g, 7, e)
        W[:, t * g:(t + 1) * g] = Wt
        C[:, t * g:(t + 1) * g] = ct
    q, sc = oracle.quant_w4g(W, g)
    assert sc.shape == (N, G)
    assert np.all(sc == np.array([np.float32(2.0 ** -e) for e in es], np.float32)[None, :])
    assert np.array_equal(q, C)


def test_quant_w4g_one_group_is_row_wise_and_groups_are_rows():
    """g = K is the row-wise quantization; and every group quantizes as a row of its own
    (the matrix [N][K] seen as [N*K/g][g]): a misplaced group index fails one of them."""
    W = workloads.weights(42, 1, 48, 512, outlier_rows=True)
    q1, s1 = oracle.quant_w4g(W, 512)
    qr, sr = oracle.quant_w4(W)
    assert np.array_equal(q1, qr) and np.array_equal(s1[:, 0].view(np.uint32), sr.view(np.uint32))
    for g in (32, 64, 128, 256):
        qg, sg = oracle.quant_w4g(W, g)
        qrows, srows = oracle.quant_w4(W.reshape(-1, g))
        assert np.array_equal(qg.reshape(-1, g), qrows)
        assert np.array_equal(sg.reshape(-1).view(np.uint32), srows.view(np.uint32))


def test_quant_w4g_invariants_and_rejections():
    W = workloads.weights(43, 1, 32, 384, outlier_rows=True)
    W[3, 128:256] = 0.0  # one all-zero group
    q, s = oracle.quant_w4g(W, 128)
    assert s[3, 1] == 0 and not q[3, 128:256].any()
    assert np.abs(q).max() <= 7
    groups = np.abs(q.reshape(32, 3, 128)).max(axis=2)
    assert np.all(groups[s > 0] == 7)
    err = np.abs(W.astype(np.float64) - q * np.repeat(s, 128, axis=1).astype(np.float64))
    assert np.all(err <= np.repeat(s, 128, axis=1) * (0.5 + 2.0 ** -20))
    with pytest.raises(oracle.OracleError):
        oracle.quant_w4g(W, 100)  # K not a multiple of g


def test_gemv_w4a8g_brute_force_exact_identity_and_bound():
    """Per-group dots by brute force; the group decomposition equals the dequantized dot
    sum_k (q s_t(k))(xq a) exactly in rationals; Y lies within the fp32 summation bound
    of that exact value."""
    g, G, N, M = 8, 4, 5, 3
    K = g * G
    W = workloads.weights(44, 1, N, K)
    X = workloads.activations(44, 2, M, K)
    q, s = oracle.quant_w4g(W, g)
    r = oracle.gemv_w4a8g(X, q, s, g)
    xq, a = r["xq"], r["a"]
    u = Fraction(1, 2 ** 24)
    for m in range(M):
        for n in range(N):
            terms = []
            for t in range(G):
                acc = sum(int(q[n, k]) * int(xq[m, k]) for k in range(t * g, (t + 1) * g))
                assert r["accg"][m, n, t] == acc
                terms.append(Fraction(acc) * Fraction(float(s[n, t])))
            exact = sum(terms) * Fraction(float(a[m]))
            deq = sum(Fraction(int(q[n, k])) * Fraction(float(s[n, k // g])) * Fraction(int(xq[m, k]))
                      for k in range(K)) * Fraction(float(a[m]))
            assert exact == deq
            bound = (G + 2) * u * sum(abs(x) for x in terms) * abs(Fraction(float(a[m])))
            assert abs(Fraction(float(r["Y"][m, n])) - exact) <= bound


def test_gemv_w4a8g_one_group_equals_row_wise_bit_for_bit():
    W = workloads.weights(45, 1, 200, 256, outlier_rows=True)
    X = workloads.activations(45, 2, 2, 256, outlier_channels=4)
    q, s = oracle.quant_w4g(W, 256)
    rg = oracle.gemv_w4a8g(X, q, s, 256)
    rr = oracle.gemv_w4a8(X, q, s[:, 0])
    assert np.array_equal(rg["Y"].view(np.uint32), rr["Y"].view(np.uint32))
    assert np.array_equal(rg["accg"][:, :, 0], rr["acc"])


def test_gemv_w4a8g_against_fp64_and_int64_matmuls():
    """At a decode shape: the per-group dots equal an int64 matmul of the codes group by
    group, and Y is within the summation bound of the fp64 value."""
    W = workloads.weights(46, 1, 96, 3584, outlier_rows=True)
    X = workloads.activations(46, 2, 1, 3584, outlier_channels=4)
    q, s = oracle.quant_w4g(W, 128)
    r = oracle.gemv_w4a8g(X, q, s, 128, nthreads=4)
    acc64 = np.einsum("mtk,ntk->mnt", r["xq"].astype(np.int64).reshape(1, 28, 128),
                      q.astype(np.int64).reshape(96, 28, 128))
    assert np.array_equal(r["accg"], acc64)
    y64, bound = oracle.w4a8g_ref64(r["accg"], s, r["a"])
    deq = (r["xq"].astype(np.float64) * r["a"].astype(np.float64)[:, None]) @ \
        (q.astype(np.float64) * np.repeat(s, 128, axis=1).astype(np.float64)).T
    assert np.allclose(y64, deq, rtol=1e-12, atol=0)
    assert np.all(np.abs(r["Y"] - y64) <= bound)
    # finer groups track the unquantized product at least as well as row-wise scales
    qr, sr = oracle.quant_w4(W)
    yr = oracle.gemv_w4a8(X, qr, sr)["Y"]
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(r["Y"] - ref) <= np.linalg.norm(yr - ref)
    rt = oracle.gemv_w4a8g(X, q, s, 128, nthreads=1)
    assert np.array_equal(rt["Y"], r["Y"])


# ------------------------------------------------- the page's two ablations --

def test_gemv_f16_ref64_brute_force_and_one_hot():
    rng = np.random.default_rng(51)
    X16 = rng.standard_normal((2, 24)).astype(np.float16)
    W16 = (rng.standard_normal((5, 24)) * 0.02).astype(np.float16)
    y = oracle.gemv_f16_ref64(X16, W16)
    for m in range(2):
        for n in range(5):
            exact = sum(Fraction(float(W16[n, k])) * Fraction(float(X16[m, k])) for k in range(24))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 80)
    e = np.zeros((1, 24), np.float16)
    e[0, 7] = 1.0
    assert np.array_equal(oracle.gemv_f16_ref64(e, W16)[0], W16[:, 7].astype(np.float64))


def test_gemv_w4f32_brute_force_and_bound():
    W = workloads.weights(52, 1, 6, 40)
    X = workloads.activations(52, 2, 3, 40)
    q, s = oracle.quant_w4(W)
    Y, Y64 = oracle.gemv_w4f32(X, q, s)
    bound = oracle.w4f32_bound(X, q, s)
    for m in range(3):
        for n in range(6):
            exact = sum(Fraction(int(q[n, k])) * Fraction(float(s[n])) * Fraction(float(X[m, k]))
                        for k in range(40))
            assert abs(Fraction(float(Y64[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 100)
            assert abs(Fraction(float(Y[m, n])) - exact) <= Fraction(float(bound[m, n]))


def test_gemv_w4f32_equals_w4a8_on_integer_activations():
    """Activations that are integers in [-127, 127] with a 127 present quantize to
    themselves with scale 1; every partial sum is then an exact fp32 integer, so the
    float-unpack path and the integer path give the same bits."""
    W = workloads.weights(53, 1, 64, 512, outlier_rows=True)
    q, s = oracle.quant_w4(W)
    rng = np.random.default_rng(53)
    X = rng.integers(-127, 128, size=(2, 512)).astype(np.float32)
    X[:, 3] = 127.0
    Yf, _ = oracle.gemv_w4f32(X, q, s)
    r = oracle.gemv_w4a8(X, q, s)
    assert np.all(r["a"] == 1.0) and np.array_equal(r["xq"], X.astype(np.int8))
    assert np.array_equal(Yf.view(np.uint32), r["Y"].view(np.uint32))


# ------------------------------------------------------------ IndexSoftmax --

def test_index_lut_values():
    """(b, c) = (5, 6.6): 32 UINT8 entries; entry 0 is exp(0) * 255, entry 1 is
    255 * e^(-6.6/31) = 206.1, the last is forced to 0; within half a unit of the
    formula evaluated with numpy's exp; non-increasing."""
    lut = oracle.index_lut(5, 6.6)
    assert lut.shape == (32,) and lut[0] == 255 and lut[1] == 206 and lut[31] == 0
    ref = 255.0 * np.exp(-6.6 * np.arange(31) / 31.0)
    assert np.all(np.abs(lut[:31] - ref) <= 0.5)
    assert np.all(np.diff(lut.astype(int)) <= 0)
    assert oracle.index_lut(4, 6.6)[15] == 0 and oracle.index_lut(4, 6.6).shape == (16,)


def test_index_softmax_closed_forms():
    # equal logits: every E is 255, P = round(255 / L), ties up (L = 2: 127.5 -> 128)
    for L, want in ((1, 255), (2, 128), (3, 85), (4, 64), (255, 1), (256, 1), (600, 0)):
        P, rs = oracle.index_softmax(np.full((1, L), -37, np.int32), 100)
        assert np.all(P == want) and rs[0] == 255 * L, L
    # one logit ahead of the rest by at least c_int: the rest clip to the last entry (0)
    A = np.array([[5, 5 + 1000, 5, -2**30]], np.int32)
    P, rs = oracle.index_softmax(A, 1000)
    assert P.tolist() == [[0, 255, 0, 0]] and rs[0] == 255
    # index rounding half up: with c_int = 62, D = 1 maps to 31/62 = 0.5 -> entry 1 and
    # D = 3 to 1.5 -> entry 2
    P, rs = oracle.index_softmax(np.array([[10, 9, 7]], np.int32), 62)
    lut = oracle.index_lut()
    assert rs[0] == 255 + int(lut[1]) + int(lut[2])


def test_index_softmax_invariants_and_float_softmax():
    rng = np.random.default_rng(61)
    d, sq, sk = 128, 0.02, 0.03
    A = rng.integers(-30000, 30000, size=(64, 777)).astype(np.int32)
    ci = oracle.index_cint(6.6, d, sq, sk)
    assert ci == 124_451  # 6.6 * sqrt(128) / 0.0006 = 124450.79...
    assert ci == round(6.6 * np.sqrt(128) / (0.02 * 0.03))
    P, rs = oracle.index_softmax(A, ci)
    P2, rs2 = oracle.index_softmax(A + np.int32(12345), ci)   # shift invariance
    assert np.array_equal(P, P2) and np.array_equal(rs, rs2)
    Pt, _ = oracle.index_softmax(A, ci, nthreads=4)
    assert np.array_equal(P, Pt)
    # each P rounds 255 E / rowSum: the row totals stay within L/2 of 255
    assert np.all(np.abs(P.astype(np.int64).sum(axis=1) - 255) <= 777 / 2)
    # the row maximum gets the largest probability
    assert np.all(P[np.arange(64), A.argmax(axis=1)] == P.max(axis=1))
    # close to the float softmax of the dequantized logits (the page reports cosine
    # 0.9991 for UINT8 probabilities) on rows as peaked as attention rows (logits of
    # standard deviation 3); on flat rows over many keys every probability is below
    # 1/510 and rounds to 0 or 1 (the 8-bit ceiling the page lists as a limitation)
    z = rng.standard_normal((64, 256)) * 3.0
    A = np.round(z * np.sqrt(d) / (sq * sk)).astype(np.int32)
    P, _ = oracle.index_softmax(A, ci)
    z = A.astype(np.float64) * sq * sk / np.sqrt(d)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    q = P / 255.0
    cos = (p * q).sum(axis=1) / np.linalg.norm(p, axis=1) / np.linalg.norm(q, axis=1)
    assert cos.mean() > 0.998 and cos.min() > 0.99


def test_int_attention_pipeline():
    rng = np.random.default_rng(62)
    Lq, Lk, d = 16, 200, 64
    Q = rng.standard_normal((Lq, d)).astype(np.float32)
    K = rng.standard_normal((Lk, d)).astype(np.float32)
    V = rng.standard_normal((Lk, d)).astype(np.float32)
    r = oracle.int_attention(Q, K, V)
    q, sq = oracle.quant_act_i8(Q.reshape(1, -1))
    k, sk = oracle.quant_act_i8(K.reshape(1, -1))
    A = q.reshape(Lq, d).astype(np.int64) @ k.reshape(Lk, d).astype(np.int64).T
    assert np.array_equal(r["A"], A)
    assert r["c_int"] == oracle.index_cint(6.6, d, sq[0], sk[0])
    assert np.array_equal(r["P"], oracle.index_softmax(r["A"], r["c_int"])[0])
    z = (Q.astype(np.float64) @ K.astype(np.float64).T) / np.sqrt(d)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    O = p @ V.astype(np.float64)
    cos = (O * r["O"]).sum() / np.linalg.norm(O) / np.linalg.norm(r["O"])
    assert cos > 0.98


def test_int_attention_pv_and_output_scale_hand_case():
    """A hand-sized case of the all-integer data flow of the IntAttention summary
    (section 方法细节: per-tensor INT8 V, UINT8 P times INT8 V in integers, then one
    dequantization; the UINT8 probabilities carry a factor 255, mechanism 3).  Two keys
    with identical rows give equal logits, so IndexSoftmax gives P = round(255 / 2) =
    128 (half up) for both.  V = [[1.0, -0.25], [0.5, 0.75]] has maxabs 1, so
    s_V = fl32(1 / 127) and its codes are 127, -32 (-31.75), 64 (63.5 rounds half to
    even) and 95 (95.25).  The integer P.V is then [128 * (127 + 64), 128 * (-32 + 95)]
    = [24448, 8064] and O = P.V * s_V / 255, within one fp32 rounding."""
    Q = np.array([[1.0, -2.0]], np.float32)
    K = np.array([[0.5, 0.25], [0.5, 0.25]], np.float32)
    V = np.array([[1.0, -0.25], [0.5, 0.75]], np.float32)
    r = oracle.int_attention(Q, K, V)
    assert r["P"].tolist() == [[128, 128]]
    s_v = np.float32(1.0) / np.float32(127.0)
    expect = np.array([24448.0, 8064.0]) * np.float64(s_v) / 255.0
    expect = expect.astype(np.float32)
    assert np.array_equal(r["O"][0], expect)
    # the float attention over two equal logits averages the rows of V: [0.75, 0.25]
    assert np.abs(r["O"][0] - np.array([0.75, 0.25])).max() < 0.01
    # O scales with V exactly (a dropped or misplaced s_V fails), and flips with its sign
    r2 = oracle.int_attention(Q, K, V * np.float32(2.0))
    assert np.array_equal(r2["O"][0], np.float32(2.0) * expect)
    r3 = oracle.int_attention(Q, K, -V)
    assert np.array_equal(r3["O"][0], -expect)
    with pytest.raises(ValueError):  # V of another head width
        oracle.int_attention(Q, K, V[:, :1])


def test_int_attention_pv_equals_an_int64_matmul():
    """On a random head the oracle's output equals the int64 product of its UINT8
    probabilities and the per-tensor INT8 codes of V (taken by the pinned activation
    quantizer), dequantized once by s_V / 255: the integer P.V is checked whole."""
    rng = np.random.default_rng(63)
    Lq, Lk, d = 12, 150, 32
    Q = rng.standard_normal((Lq, d)).astype(np.float32)
    K = rng.standard_normal((Lk, d)).astype(np.float32)
    V = rng.standard_normal((Lk, d)).astype(np.float32)
    r = oracle.int_attention(Q, K, V)
    v, sv = oracle.quant_act_i8(V.reshape(1, -1))
    acc = r["P"].astype(np.int64) @ v.reshape(Lk, d).astype(np.int64)
    assert np.abs(acc).max() < 2 ** 31
    O = (acc.astype(np.float64) * np.float64(sv[0]) / 255.0).astype(np.float32)
    assert np.array_equal(r["O"].view(np.uint32), O.view(np.uint32))
    # the probabilities of each row sum to 255 within half a unit per key
    assert np.all(np.abs(r["P"].astype(np.int64).sum(axis=1) - 255) <= Lk // 2)


# ------------------------------------------------------------ W8 weights --

def test_quant_w8_closed_form_rows():
    rng = np.random.default_rng(31)
    W, c = _pow2_rows(rng, 5, 50, 127, 10)   # maxabs/127 = 2^-10, an exact half
    q, s16 = oracle.quant_w8(W)
    assert np.all(s16 == np.float16(2.0 ** -10).view(np.uint16))
    assert np.array_equal(q, c)


def test_quant_w8_codes_use_the_stored_f16_scale():
    # For a normal binary16 scale the relative rounding error is below 2^-11, so
    # maxabs / s16 stays below 127.5.  In the subnormal range (maxabs/127 < 2^-14)
    # the stored scale can be much coarser: find maxabs values whose scale rounds
    # DOWN there; their largest entry then divides to more than 127.5 and clamps.
    cand = np.float32(1e-4) + np.arange(4000, dtype=np.float32) * np.float32(1e-7)
    s32 = cand / np.float32(127)
    s16f = s32.astype(np.float16).astype(np.float32)
    down = cand[(cand / s16f) > np.float32(127.5)]
    assert down.size > 0
    m = down[0]
    W = np.array([[m, -m / 2, m / 3, 0.0]], np.float32)
    q, s16 = oracle.quant_w8(W)
    sf = oracle.f32_from_f16(s16)[0]
    assert s16[0] == np.float32(m / np.float32(127)).astype(np.float16).view(np.uint16)
    assert q[0, 0] == 127
    assert q[0, 1] == np.rint(np.float32(-m / 2) / sf)
    assert q[0, 1] != np.rint(np.float32(-m / 2) / (m / np.float32(127)))


def test_quant_w8_underflowing_scale_is_a_zero_row():
    W = np.full((1, 16), 1e-7, np.float32)   # 1e-7/127 is below half the smallest half
    q, s16 = oracle.quant_w8(W)
    assert s16[0] == 0 and not q.any()


def test_quant_w8_invariants():
    W = workloads.weights(32, 1, 64, 256)
    q, s16 = oracle.quant_w8(W)
    sf = oracle.f32_from_f16(s16).astype(np.float64)
    assert np.abs(q).max() <= 127
    assert np.all(np.abs(q).max(axis=1) >= 126)
    err = np.abs(W - q * sf[:, None])
    inside = np.abs(W / sf[:, None]) <= 127
    assert np.all(err[inside] <= (sf[:, None] * (0.5 + 2.0 ** -20) * np.ones_like(err))[inside])


# ------------------------------------------------------------ W8A16 linear --

def test_gemv_w8a16_ref64_brute_force_and_one_hot():
    W = workloads.weights(41, 1, 7, 16)
    q, s16 = oracle.quant_w8(W)
    X16 = workloads.activations(41, 2, 2, 16, dtype=np.float16)
    y = oracle.gemv_w8a16_ref64(X16, q, s16)
    sf = [Fraction(float(v)) for v in s16.view(np.float16)]
    xf = X16.astype(np.float64)
    for m in range(2):
        for n in range(7):
            exact = sum(Fraction(int(q[n, k])) * sf[n] * Fraction(float(xf[m, k])) for k in range(16))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(16, 2 ** 52) + Fraction(1, 2 ** 80)
    X1 = np.zeros((1, 16), np.float16)
    X1[0, 5] = np.float16(-2.0)
    y1 = oracle.gemv_w8a16_ref64(X1, q, s16)
    assert np.array_equal(y1[0], -2.0 * q[:, 5] * s16.view(np.float16).astype(np.float64))


def test_gemv_w8a16_sign_and_threads():
    W = workloads.weights(42, 1, 100, 128)
    q, s16 = oracle.quant_w8(W)
    X16 = workloads.activations(42, 2, 3, 128, dtype=np.float16)
    y = oracle.gemv_w8a16_ref64(X16, q, s16)
    assert np.array_equal(oracle.gemv_w8a16_ref64(-X16, q, s16), -y)
    assert np.array_equal(oracle.gemv_w8a16_ref64(X16, q, s16, nthreads=4), y)


def test_w8a16_cosine_against_unquantized_weights():
    """ChatGLM2-6B W8A16 write-up, section 2: per-channel INT8 keeps the output's
    cosine similarity to F16 above 99%.  Checked on a slice of the 4096 x 27392 linear."""
    K, N = 4096, 27392
    rows = np.arange(0, N, 16)[:1024]
    W = workloads.weight_rows(2, workloads.tensor_id("chatglm2", 0), N, K, rows)
    X16 = workloads.activations(2, workloads.tensor_id("chatglm2", 1), 1, K, dtype=np.float16)
    q, s16 = oracle.quant_w8(W)
    y = oracle.gemv_w8a16_ref64(X16, q, s16, nthreads=4)[0]
    yf = X16.astype(np.float64)[0] @ W.astype(np.float64).T
    cos = float(y @ yf / np.linalg.norm(y) / np.linalg.norm(yf))
    assert cos > 0.99
    assert cos > 0.9999  # per-channel INT8 at these magnitudes loses ~1e-5


# ------------------------------------------------------ page storage figures --

def test_page_storage_figures():
    g = json.load(open(os.path.join(GOLDEN, "p2_chatglm2_storage.json")))
    MiB = 2.0 ** 20
    elems = g["R_rows"] * g["R_cols"]
    assert round(elems * 2 / MiB) == g["weight_f16_MB"]     # f16 weights: 214.0 MiB
    assert round(elems * 1 / MiB) == g["weight_int8_MB"]    # INT8 weights: 107.0 MiB
    scale = g["scale_elems"] * g["scale_dtype_bytes"] / MiB
    assert round(scale, 3) == g["scale_MB"]                 # 4096 x f16 = 0.0078 MiB
    # Our layout keeps one f16 scale per OUTPUT channel (27392 of them): still
    # negligible next to the INT8 weights, as the page says of its scale.
    ours = g["R_cols"] * 2
    assert ours == 54784 and ours / elems < 5e-4
