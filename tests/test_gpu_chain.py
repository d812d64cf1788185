"""The decode-step chain (28 layers of seven W4A8 linears plus the lm_head in one HIP
graph) and its fused form (q|k|v and gate|up as single linears), on an MI355X.

Bars: graph replays equal eager launches bit for bit (every W4A8 step is exact up to
the fixed fp32 epilogue); sampled output rows of every linear equal the oracle within
1e-6 relative error with int32 sums exact; a fused projection's output is the
concatenation of the separate projections' outputs bit for bit, and the packed
weights of a concatenation along N are the concatenation of the packed parts.
"""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
from bit_weight_quantized_load_amd import chain
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

SEED = wl.QWEN7B_W4A8["seed"]
LM_N = 19008  # the lm_head share of one GPU at 8-way tensor parallelism


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    packed, sample = {}, {}
    for name, K, N in wl.QWEN7B_LINEARS:
        W = wl.weights(SEED, wl.tensor_id(name, 0), N, K, outlier_rows=True)
        packed[name] = qw.quantize_pack_w4(torch.from_numpy(W).cuda())
        rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                         np.random.default_rng(K + N).choice(N, 48, replace=False)]))
        sample[name] = (rows, W[rows])
    W = wl.weights(SEED, wl.tensor_id("lm_head", 0), LM_N, wl.HIDDEN)
    lm = qw.quantize_pack_w4(torch.from_numpy(W).cuda())
    rows = np.unique(np.concatenate([np.arange(8), np.arange(LM_N - 8, LM_N)]))
    sample["lm_head"] = (rows, W[rows])
    xh = wl.activations(SEED, wl.tensor_id("q_proj", 1), 1, wl.HIDDEN, outlier_channels=4)
    xi = wl.activations(SEED, wl.tensor_id("down_proj", 1), 1, wl.INTERMEDIATE, outlier_channels=4)
    torch.cuda.synchronize()
    return packed, lm, xh, xi, sample


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_chain_graph_replays_match_eager_and_oracle(layer):
    packed, lm, xh, xi, sample = layer
    c = chain.DecodeChain(packed, lm, torch.from_numpy(xh).cuda(), torch.from_numpy(xi).cuda(),
                          layers=2)
    assert c.launches_per_token == 2 * 7 + 1
    c.run()
    eager = {k: host(v).copy() for k, v in c.out.items()}
    # sampled rows of every linear against the oracle
    for name, (rows, Ws) in sample.items():
        say("chain oracle", name)
        x = xi if name == "down_proj" else xh
        q, s = oracle.quant_w4(Ws)
        ref = oracle.gemv_w4a8(x, q, s)
        y = eager[name][:, rows]
        rel = np.abs(y - ref["Y"]) / np.maximum(np.abs(ref["Y"]), 1e-30)
        assert rel.max() <= 1e-6, (name, rel.max())
    g = c.capture()
    for rep in range(3):
        for v in c.out.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, v in c.out.items():
            assert np.array_equal(host(v).view(np.uint32), eager[k].view(np.uint32)), (rep, k)
        c.run()  # eager work between replays
        torch.cuda.synchronize()


def test_fused_projections_equal_the_separate_ones(layer):
    packed, lm, xh, xi, sample = layer
    # packing the concatenated weights gives the concatenated packed buffers
    parts = [("q_proj", 64), ("k_proj", 32), ("v_proj", 36)]
    Ws = [wl.weights(SEED, wl.tensor_id(n, 0), rows, wl.HIDDEN, outlier_rows=True)
          for n, rows in parts]
    cat_packed = qw.quantize_pack_w4(torch.from_numpy(np.concatenate(Ws)).cuda())
    fused = chain.fuse_along_n([qw.quantize_pack_w4(torch.from_numpy(W).cuda()) for W in Ws])
    assert torch.equal(cat_packed[0], fused[0]) and torch.equal(cat_packed[1], fused[1])
    with pytest.raises(ValueError):
        chain.fuse_along_n([qw.quantize_pack_w4(torch.from_numpy(Ws[0][:6]).cuda())])

    xh_d, xi_d = torch.from_numpy(xh).cuda(), torch.from_numpy(xi).cuda()
    sep = chain.DecodeChain(packed, None, xh_d, xi_d, layers=1)
    fus = chain.DecodeChain(packed, None, xh_d, xi_d, layers=1, fused=True)
    assert fus.launches_per_token == 4
    assert fus.bytes_per_token < sep.bytes_per_token  # X read and quantized fewer times
    sep.run()
    g = fus.capture()
    g.replay()
    o = {k: host(v) for k, v in sep.out.items()}
    f = {k: host(v) for k, v in fus.out.items()}
    qkv = np.concatenate([o["q_proj"], o["k_proj"], o["v_proj"]], axis=1)
    gate_up = np.concatenate([o["gate_proj"], o["up_proj"]], axis=1)
    assert np.array_equal(f["qkv_proj"].view(np.uint32), qkv.view(np.uint32))
    assert np.array_equal(f["gate_up_proj"].view(np.uint32), gate_up.view(np.uint32))
    assert np.array_equal(f["o_proj"].view(np.uint32), o["o_proj"].view(np.uint32))
    assert np.array_equal(f["down_proj"].view(np.uint32), o["down_proj"].view(np.uint32))


@pytest.mark.parametrize("group", ["qkv_proj", "gate_up_proj"])
def test_fused_projection_matches_the_oracle(layer, group):
    """The fused q|k|v (3584 -> 4608) and gate|up (3584 -> 37888) launches, one
    activation quantization each, against the oracle on the concatenated weights: the
    activation codes and scale, every int32 sum and every output (the page's next step
    of removing the repeated quantization of the QKV and MLP projections, "Jetson Orin
    AGX 上的 INT4 量化推理实践", section 后续优化方向)."""
    packed, lm, xh, xi, sample = layer
    parts = dict(chain.FUSED_GROUPS)[group]
    W = np.concatenate([wl.weights(SEED, wl.tensor_id(p, 0), dict((n, N) for n, _, N in
                                                                  wl.QWEN7B_LINEARS)[p],
                                   wl.HIDDEN, outlier_rows=True) for p in parts])
    N = W.shape[0]
    say("fused vs oracle", group, N)
    q, s = oracle.quant_w4(W)
    del W
    ref = oracle.gemv_w4a8(xh, q, s, nthreads=oracle.num_threads())
    wq, sc = chain.fuse_along_n([packed[p] for p in parts])
    assert np.array_equal(host(sc).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(host(qw.w4_codes(wq, N, wl.HIDDEN)), q)
    xd = torch.from_numpy(xh).cuda()
    out = qw.gemv_w4a8_debug(xd, wq, sc)
    assert np.array_equal(host(out["xq"]), ref["xq"])
    assert np.array_equal(host(out["a"]).view(np.uint32), ref["a"].view(np.uint32))
    assert np.array_equal(host(out["acc"]), ref["acc"])
    assert np.array_equal(host(out["Y"]).view(np.uint32), ref["Y"].view(np.uint32))
    # the fused chain's launch of this group gives the same bits
    fus = chain.DecodeChain(packed, None, xd, torch.from_numpy(xi).cuda(), layers=1, fused=True)
    fus.run()
    assert np.array_equal(host(fus.out[group]).view(np.uint32), ref["Y"].view(np.uint32))
