"""Parity of the IndexSoftmax kernel (the integer softmax of the IntAttention summary,
section 基准/方法设计) with the CPU oracle: integer work, so bit-exact, on logits over the
whole int32 range (the row maximum minus a logit overflows int32 and must not wrap),
attention-like peaked rows, constant rows, one-element rows, ragged lengths up to 16384,
and b = 4, 5, 6 with thresholds from 1 to 2^31 - 1 (on both sides of the bound of the
exact multiply-high index, c_int < 2^24 and c_int (2n + 1) < 2^31, and a power of two).
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


def logits(kind, rows, L, seed):
    rng = np.random.default_rng(seed)
    if kind == "full":
        return rng.integers(-2**31, 2**31, size=(rows, L), dtype=np.int64).astype(np.int32)
    if kind == "peaked":  # attention-like: logits of standard deviation 3 at scales 0.02, 0.03
        z = rng.standard_normal((rows, L)) * 3.0
        return np.round(z * np.sqrt(128) / (0.02 * 0.03)).astype(np.int32)
    if kind == "const":
        return np.full((rows, L), -17, np.int32)
    raise ValueError(kind)


CASES = [(3, 1), (5, 7), (64, 1000), (37, 1024), (16, 4096), (9, 4097), (4, 16384), (6, 3),
         (2, 10001)]


@pytest.mark.parametrize("rows,L", CASES)
@pytest.mark.parametrize("kind", ["full", "peaked", "const"])
def test_index_softmax_bit_exact(rows, L, kind):
    print("index_softmax", kind, rows, L, flush=True)
    A = logits(kind, rows, L, rows * 1000 + L)
    Ad = dev(A)
    for (b, ci) in ((5, 124451), (5, 1), (4, 62), (6, 2**31 - 1), (5, 3 * 10**6), (6, 2**20),
                    (4, 2**24 - 1), (4, 2**24)):
        P = host(qw.index_softmax(Ad, ci, b=b, c=6.6))
        Po, rs = oracle.index_softmax(A, ci, b=b, c=6.6)
        assert np.array_equal(P, Po), (b, ci)


def test_index_cint_matches_the_oracle():
    for (c, d, sq, sk) in ((6.6, 128, 0.02, 0.03), (5.5, 64, 0.1, 0.007), (7.7, 256, 1e-3, 2e-3)):
        assert qw.index_cint(c, d, sq, sk) == oracle.index_cint(c, d, sq, sk)
