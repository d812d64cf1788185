"""Error bounds shared by the GPU parity tests.

W8A16 has more than one correct output: the kernels add the K exact products q * x in
fp32 in an order of their choosing (the ChatGLM2-6B W8A16 write-up, section 4, fixes the
computation, not the order).  The bar is the relative L2 error of 1e-3 over the whole
output against the fp64 dequantize-then-multiply reference, and per element the fp32
summation bound plus the final f16 rounding, which any valid order meets and a
mis-indexed chunk or row does not.
"""
import numpy as np

import oracle

W8A16_RL2 = 1e-3


def rel_l2(y, y64):
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(y - y64) / max(np.linalg.norm(y64), 1e-300))


def half_ulp16(v):
    """Half a binary16 ulp at magnitude |v| (2^-25 in the subnormal range)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.maximum(v, 2.0 ** -14))
    return np.ldexp(1.0, e - 12)


def w8a16_bound(X16, q, s16):
    """Per-element bound of a W8A16 output around the exact value: the kernel sums the
    K exact products q*x in fp32 in an order of its choosing (each addition rounds by at
    most 2^-24 relative, so the sum is within (K - 1) * 2^-24 * sum|q*x|), multiplies by
    the f16 scale (one more rounding) and rounds to f16 (half an ulp).  sum|q*x| is
    taken in fp32 from exactly representable |q| and |x| and padded by 0.1%."""
    K = X16.shape[1]
    s = oracle.f32_from_f16(np.asarray(s16)).astype(np.float64)
    absdot = np.abs(X16.astype(np.float32)) @ np.abs(q.astype(np.float32)).T
    return (K + 2) * 2.0 ** -24 * absdot.astype(np.float64) * s[None, :] * 1.001


def check_w8a16(y, X16, q, s16, y64):
    """The W8A16 bars: relative L2 error <= 1e-3 over the whole output, and per element
    |y - y64| <= half an f16 ulp + the fp32 summation bound (any valid order of the
    fp32 sums meets it; a mis-indexed chunk or row does not)."""
    y = np.asarray(y, np.float32).astype(np.float64)
    assert rel_l2(y, y64) <= W8A16_RL2
    bound = half_ulp16(np.maximum(np.abs(y), np.abs(y64))) + w8a16_bound(X16, q, s16)
    err = np.abs(y - y64)
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float((err - bound).max()), np.argwhere(bad)[:4])
