"""Seeded synthetic inputs and workload shapes for the weight-quantized decode linear.

This module is shared by the oracle's tests, the GPU tests and the benchmark.  It
holds no step of the method itself (no quantization, packing or dot product): it
only draws fp32/fp16 tensors with the shapes and value distributions of the
decode workloads, deterministically from a seed.

Recipe (the same everywhere):

* A tensor is drawn in row blocks of ``ROW_BLOCK`` rows.  Block ``b`` of tensor
  ``tid`` under seed ``seed`` comes from numpy's PCG64 seeded with
  ``SeedSequence([seed, tid, b])``, as float32 standard normals, times a float32
  standard deviation (one fp32 rounding).  Blocks are independent, so any row can be
  regenerated alone and the result does not depend on the thread count.
* Weight outliers: ``N // 100`` distinct rows (PCG64 under
  ``SeedSequence([seed, tid, OUTLIER_STREAM])``, choice without replacement) are
  multiplied by 8 (exact in fp32).
* Activation outliers: ``n`` distinct channels k chosen the same way are
  multiplied by 20 in fp32.
* fp16 activations are the fp32 draw rounded to binary16 (round half to even).

Workload shapes come from the two models the pages measure: a Qwen-7B-class
decoder (hidden 3584, intermediate 18944, vocabulary 152064, 28 layers, grouped
k/v projections of width 512) and ChatGLM2-6B's 4096 x 27392 linear.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BLOCK = 1024
OUTLIER_STREAM = 0x6F75746C  # "outl"

# ---------------------------------------------------------------- shapes -----
HIDDEN = 3584
INTERMEDIATE = 18944
VOCAB = 152064
LAYERS = 28
KV_WIDTH = 512

# (name, K, N) of the seven linears of one Qwen-7B-class decoder layer.
QWEN7B_LINEARS = (
    ("q_proj", HIDDEN, HIDDEN),
    ("k_proj", HIDDEN, KV_WIDTH),
    ("v_proj", HIDDEN, KV_WIDTH),
    ("o_proj", HIDDEN, HIDDEN),
    ("gate_proj", HIDDEN, INTERMEDIATE),
    ("up_proj", HIDDEN, INTERMEDIATE),
    ("down_proj", INTERMEDIATE, HIDDEN),
)
LM_HEAD = ("lm_head", HIDDEN, VOCAB)

# Named workloads.  Each config draws with its own seed.
TINY_W4A8 = {"workload": "tiny_w4a8", "M": 1, "K": 256, "N": 512, "seed": 0}
QWEN7B_W4A8 = {"workload": "qwen7b_linears_w4a8", "M": 1, "seed": 1,
               "weight_outlier_rows": True, "act_outlier_channels": 4}
CHATGLM2_W8A16 = {"workload": "chatglm2_w8a16", "M": 1, "K": 4096, "N": 27392, "seed": 2}
LMHEAD_W4A8 = {"workload": "lm_head_w4a8", "M": 1, "K": HIDDEN, "N": VOCAB, "seed": 3}
SKINNY = {"workload": "skinny_sweep", "K": 4096, "N": 27392, "Ms": (1, 4, 16, 64, 512), "seed": 4}
# The down projection of the Qwen-7B-class layer (long K) at a few rows of X.
LONG_K = {"workload": "long_k_sweep_18944x3584", "K": INTERMEDIATE, "N": HIDDEN,
          "Ms": (1, 2, 4, 16), "seed": 5}
# The headline decode linear: the gate/up projection of the Qwen-7B-class layer.
HEADLINE = {"workload": "qwen7b_gate_up_3584x18944", "M": 1, "K": HIDDEN, "N": INTERMEDIATE}

WEIGHT_STD = 0.02


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _block(seed: int, tid: int, b: int, rows: int, K: int, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b])))
    z = g.standard_normal((rows, K), dtype=np.float32)
    z *= np.float32(std)
    return z


def normal_matrix(seed: int, tid: int, R: int, K: int, std: float = 1.0) -> np.ndarray:
    """float32 [R][K] with entries std * N(0, 1), drawn block by block."""
    out = np.empty((R, K), np.float32)
    nblk = (R + ROW_BLOCK - 1) // ROW_BLOCK

    def fill(b):
        r0 = b * ROW_BLOCK
        r1 = min(R, r0 + ROW_BLOCK)
        out[r0:r1] = _block(seed, tid, b, r1 - r0, K, std)

    if nblk <= 1 or R * K < (1 << 22):
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def normal_rows(seed: int, tid: int, R: int, K: int, rows, std: float = 1.0) -> np.ndarray:
    """Rows ``rows`` of ``normal_matrix(seed, tid, R, K, std)``, drawn without the rest."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, K), np.float32)
    cache = {}
    for i, r in enumerate(rows):
        b = int(r) // ROW_BLOCK
        if b not in cache:
            nrows = min(R, (b + 1) * ROW_BLOCK) - b * ROW_BLOCK
            cache[b] = _block(seed, tid, b, nrows, K, std)
        out[i] = cache[b][int(r) - b * ROW_BLOCK]
    return out


def pick_distinct(seed: int, tid: int, n_total: int, count: int) -> np.ndarray:
    """``count`` distinct indices in [0, n_total), sorted."""
    if count <= 0:
        return np.zeros((0,), np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, OUTLIER_STREAM])))
    return np.sort(g.choice(n_total, size=count, replace=False)).astype(np.int64)


def weight_outlier_rows(seed: int, tid: int, N: int) -> np.ndarray:
    return pick_distinct(seed, tid, N, N // 100)


def weights(seed: int, tid: int, N: int, K: int, outlier_rows: bool = False,
            std: float = WEIGHT_STD) -> np.ndarray:
    """fp32 [N][K] ~ N(0, std); with ``outlier_rows`` 1% of the rows are scaled 8x."""
    W = normal_matrix(seed, tid, N, K, std)
    if outlier_rows:
        W[weight_outlier_rows(seed, tid, N)] *= np.float32(8.0)
    return W


def weight_rows(seed: int, tid: int, N: int, K: int, rows, outlier_rows: bool = False,
                std: float = WEIGHT_STD) -> np.ndarray:
    """Rows ``rows`` of ``weights(...)`` without drawing the whole matrix."""
    rows = np.asarray(rows, dtype=np.int64)
    W = normal_rows(seed, tid, N, K, rows, std)
    if outlier_rows:
        hot = set(weight_outlier_rows(seed, tid, N).tolist())
        for i, r in enumerate(rows):
            if int(r) in hot:
                W[i] *= np.float32(8.0)
    return W


def activations(seed: int, tid: int, M: int, K: int, outlier_channels: int = 0,
                dtype=np.float32) -> np.ndarray:
    """[M][K] ~ N(0, 1); ``outlier_channels`` distinct channels scaled 20x.

    ``dtype`` float32, or float16 (the fp32 draw rounded to binary16)."""
    X = normal_matrix(seed, tid, M, K, 1.0)
    if outlier_channels:
        X[:, pick_distinct(seed, tid, K, outlier_channels)] *= np.float32(20.0)
    if dtype == np.float16:
        return X.astype(np.float16)
    return X


# Tensor ids: one per (linear, role).  Role 0 = weight, 1 = activation.
def tensor_id(name: str, role: int) -> int:
    names = [n for n, _, _ in QWEN7B_LINEARS] + ["lm_head", "tiny", "chatglm2", "skinny", "headline_w8"]
    return 16 * (names.index(name) + 1) + role
