#!/usr/bin/env python3
"""Benchmark of the weight-quantized decode linear on one MI355X.

One step is the decode linear at the headline shape M=1, K=3584, N=18944 (the
gate/up projection of a Qwen-7B-class layer) in both variants: one W4A8 GEMV (with
its fused activation quantization) and one W8A16 GEMV.  Weight packing is load-time
work and stays outside the timed region.  The packed weights are replicated into
enough distinct copies (rotated step by step) that every step reads them from HBM,
not from the 256 MB last-level cache.

Printed: ONE JSON line with `value` = algorithmic bytes of both GEMVs / time per
step (GB/s), per-kernel microseconds and GB/s (also, outside the step, of the group-wise
INT4 variant and of the INT4 page's two ablations -- an FP16 GEMV and weight-only INT4
unpacked to float -- on the same shape, and of IndexSoftmax on 8192 x 4096 int32
attention logits), the roofline of the dominant kernel
(per-launch algorithmic bytes / average launch time from HIP events), the CPU
oracle timed on this host on the same inputs, and the linear-layer time per token
of the 28-layer decode-step chain in one HIP graph (unfused and with q|k|v and
gate|up fused).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8/W8A16 GEMV µs and HBM GB/s (% of peak), M=1 K=3584 N=18944"
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1.5e9  # > 256 MB last-level cache, several times over
# At most this many rotated copies of one buffer: shapes below 1.5 GB / 1024 (the tiny
# and k/v linears, under 1.5 MB) are launch-bound, and a graph of tens of thousands of
# launches per timing adds nothing.
MAX_COPIES = 1024


def bytes_w4a8(M, N, K):
    """Algorithmic bytes: 0.5 B per INT4 weight, 4 B per scale, X element and Y element."""
    return N * K // 2 + 4 * N + 4 * M * K + 4 * M * N


def bytes_w4a8g(M, N, K, g):
    """Algorithmic bytes of the group-wise variant: 0.5 B per INT4 weight, 4 B per group
    scale (N * K / g of them), 4 B per X and Y element."""
    return N * K // 2 + 4 * N * (K // g) + 4 * M * K + 4 * M * N


def bytes_w8a16(M, N, K):
    """Algorithmic bytes: 1 B per INT8 weight, 2 B per f16 scale, X element and Y element."""
    return N * K + 2 * N + 2 * M * K + 2 * M * N


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and whitespace removed) of the sources that define the
    kernel and choose its launch shape."""
    import re

    csrc = os.path.join(ROOT, "bit_weight_quantized_load_amd", "csrc")
    files = ["common.hpp", "kernels.hpp", "gemv_shapes.hpp"]
    files += ["gemv_w4a8.hip", "w4a8_prod.hpp"] if kernel == "gemv_w4a8" else ["gemv_w8a16.hip"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f)) as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def host_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, X, X16, seconds, b_step):
    """The oracle, as it stands, on this host: one step is W4A8 (activation quantization,
    integer GEMV, epilogue) plus the fp64 W8A16 reference on the headline inputs.  At all
    of the host's threads: the median of 5 runs of `reps` steps each, `reps` chosen so
    the 5 runs take about `seconds`; at one thread: the median of 5 single steps.  Weight
    quantization is load-time work on both sides and is not timed."""
    import statistics

    import oracle

    q4, s4 = oracle.quant_w4(W)
    q8, s8 = oracle.quant_w8(W)
    nt = host_threads()

    def step(n):
        oracle.gemv_w4a8(X, q4, s4, nthreads=n)
        oracle.gemv_w8a16_ref64(X16, q8, s8, nthreads=n)

    def run(n, reps):
        t0 = time.perf_counter()
        for _ in range(reps):
            step(n)
        return (time.perf_counter() - t0) / reps

    step(nt)
    reps = max(1, int(seconds / 5 / max(run(nt, 1), 1e-4)))
    t_all = statistics.median(run(nt, reps) for _ in range(5))
    t_one = statistics.median(run(1, 1) for _ in range(5))
    return {"value": round(b_step / t_all / 1e9, 4), "unit": "GB/s", "cores": nt,
            "kind": "oracle",
            "sample": "the full step (W4A8 + fp64 W8A16 reference, M=1 K=3584 N=18944): median "
                      "of 5 runs of %d steps on %d OpenMP threads; 1 thread: median of 5 steps"
                      % (reps, nt),
            "value_1_thread": round(b_step / t_one / 1e9, 4),
            "ms_per_step": {"1_thread": round(t_one * 1e3, 3), "%d_threads" % nt: round(t_all * 1e3, 3)},
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def _pmc_per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} of one counter from a rocprofv3 --pmc CSV
    (values reported per dimension are summed per dispatch)."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if (r.get("Counter_Name") or r.get("Counter-Name")) != counter:
                continue
            name = r.get("Kernel_Name") or r.get("Kernel-Name")
            disp = r.get("Dispatch_Id") or r.get("Dispatch-Id")
            per[name][disp] += float(r.get("Counter_Value") or r.get("Counter-Value"))
    return {k: list(v.values()) for k, v in per.items()}


# The kernel instances the headline step runs (built-in launch shapes at M=1, K=3584,
# N=18944); the counters are read for these names exactly.
HEADLINE_KERNELS = {"gemv_w4a8": "k_gemv_w4a8_prod<7, 8, 2, 1, 0, false>",
                    "gemv_w8a16": "k_gemv_w8a16_flight<7, 1, 4>"}


def write_traffic(fetch_copy, write_copy, fetch_bench, write_bench, copy_bytes, commands):
    """HBM bytes per launch of both GEMVs from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch, each on a plain device copy of copy_bytes and on this
    benchmark), each counter scaled by copy_bytes / (its median reading on the copy);
    written to profiles/traffic_<kernel>_<workload>.json with the hash of the kernel
    sources they were taken on."""
    import statistics

    import workloads as wl

    def median_of(path, counter, key):
        vals = [v for k, vs in _pmc_per_dispatch(path, counter).items() if key in k for v in vs]
        if not vals:
            raise SystemExit("no %s dispatches of %s in %s" % (counter, key, path))
        return statistics.median(vals)

    fc = median_of(fetch_copy, "FETCH_SIZE", "copyBuffer")
    wc = median_of(write_copy, "WRITE_SIZE", "copyBuffer")
    f_scale, w_scale = copy_bytes / 1024.0 / fc, copy_bytes / 1024.0 / wc
    c = wl.HEADLINE
    M, K, N = c["M"], c["K"], c["N"]
    for kernel, algo in (("gemv_w4a8", bytes_w4a8(M, N, K)), ("gemv_w8a16", bytes_w8a16(M, N, K))):
        fk = median_of(fetch_bench, "FETCH_SIZE", HEADLINE_KERNELS[kernel])
        wk = median_of(write_bench, "WRITE_SIZE", HEADLINE_KERNELS[kernel])
        hbm = int(round((fk * f_scale + wk * w_scale) * 1024))
        out = {"kernel": kernel, "workload": c["workload"],
               "kernel_source_sha": kernel_source_hash(kernel),
               "fetch_size_kib": fk, "write_size_kib": wk,
               "fetch_scale": round(f_scale, 6), "write_scale": round(w_scale, 6),
               "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": algo,
               "ratio": round(hbm / algo, 4),
               "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib": fc, "write_size_kib": wc},
               "commands": commands}
        path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, c["workload"]))
        with open(path, "w") as fh:
            json.dump(out, fh, indent=1)
        print(json.dumps(out))


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


# Untimed replays before each timed measurement run for at least this long: after host
# work the GPU clock is low, and the first milliseconds of a measurement otherwise run
# slower (the first of several kernels timed in a row read up to 15% slow).
WARM_S = 0.02


def graph_us(torch, fn, n, reps=3):
    """Per-launch microseconds of fn(0), ..., fn(n - 1) captured in one HIP graph:
    untimed replays for at least WARM_S seconds, then the median of `reps` replays timed
    with HIP events on the stream the graph runs on.  Callers pass n >= the number of
    rotated copies, so every copy is read in each replay."""
    import statistics

    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARM_S:
            break
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / n)
    del g
    return statistics.median(ts)


class ReadPool:
    """One large device buffer whose disjoint slices serve as rotated sources of the bare
    streaming read: slices of B bytes at 4 KB-aligned offsets, as many as fit."""

    def __init__(self, torch, nbytes=int(2 * ROTATE_BYTES)):
        self.torch = torch
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.buf.fill_(0x5A)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        self.sink = torch.empty(max(cus, 1024), dtype=torch.int32, device="cuda")

    def time_us(self, qw, B, launches):
        """Bare read of B bytes (rounded up to 16), rotated over the pool's slices."""
        B = -(-B // 16) * 16
        step = -(-B // 4096) * 4096
        R = max(1, min(MAX_COPIES, self.buf.numel() // step))
        srcs = [self.buf[i * step:i * step + B] for i in range(R)]
        n = max(launches, R)
        return graph_us(self.torch, lambda i: qw.stream_read(srcs[i % R], self.sink), n), R


def w4_config_times(qw, torch, W, X, pool, launches):
    """W4A8 at M = 1 on the given weights (fp32 host arrays): (us, weight copies, bare-read
    us of the same algorithmic bytes)."""
    N, K = W.shape
    Wq, s = qw.quantize_pack_w4(torch.from_numpy(W).cuda())
    R = max(2, min(MAX_COPIES, math.ceil(ROTATE_BYTES / Wq.numel())))
    copies = [(Wq, s)] + [(Wq.clone(), s.clone()) for _ in range(R - 1)]
    Xd = torch.from_numpy(X).cuda()
    Y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    t = graph_us(torch, lambda i: qw.gemv_w4a8(Xd, copies[i % R][0], copies[i % R][1], out=Y),
                 max(launches, R))
    tb, _ = pool.time_us(qw, bytes_w4a8(1, N, K), launches)
    del copies, Wq, s
    return t, R, tb


def w8_config_times(qw, torch, W, X16, pool, launches):
    N, K = W.shape
    Wq, s = qw.quantize_pack_w8(torch.from_numpy(W).cuda())
    R = max(2, min(MAX_COPIES, math.ceil(ROTATE_BYTES / Wq.numel())))
    copies = [(Wq, s)] + [(Wq.clone(), s.clone()) for _ in range(R - 1)]
    Xd = torch.from_numpy(X16).cuda()
    Y = torch.empty((1, N), dtype=torch.float16, device="cuda")
    t = graph_us(torch, lambda i: qw.gemv_w8a16(Xd, copies[i % R][0], copies[i % R][1], out=Y),
                 max(launches, R))
    tb, _ = pool.time_us(qw, bytes_w8a16(1, N, K), launches)
    del copies, Wq, s
    return t, R, tb


def oracle_ms(fn, runs):
    """Median wall time of `runs` calls of fn(), in ms."""
    import statistics

    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append((time.perf_counter() - t0) * 1e3)
    return statistics.median(ts)


def configs_measurement(qw, wl, torch, pool, launches, with_oracle):
    """Each decode linear of the workloads at M = 1 on its own: the tiny config, the seven
    Qwen-7B projections (one line per distinct shape), the fused q|k|v and gate|up
    launches, the lm_head and ChatGLM2's W8A16 linear.  Per line: GPU us (HIP events,
    weight copies rotated past the cache), algorithmic bytes, GB/s and fraction of
    8 TB/s, the bare streaming read of the same number of bytes (the ceiling a
    weight-streaming kernel of that size meets on this GPU), and the oracle's wall time
    on this host at 1 thread and at all threads (median of 3, of 1 for the lm_head at
    1 thread)."""
    import oracle

    nt = host_threads()
    seed = wl.QWEN7B_W4A8["seed"]
    lines = {}

    def qwen(name, rows=None):
        K, N = [(k, n) for nm, k, n in wl.QWEN7B_LINEARS if nm == name][0]
        return wl.weights(seed, wl.tensor_id(name, 0), N, K, outlier_rows=True)

    xh = wl.activations(seed, wl.tensor_id("q_proj", 1), 1, wl.HIDDEN, outlier_channels=4)
    xi = wl.activations(seed, wl.tensor_id("down_proj", 1), 1, wl.INTERMEDIATE, outlier_channels=4)
    c0 = wl.TINY_W4A8
    c3 = wl.LMHEAD_W4A8
    c2 = wl.CHATGLM2_W8A16
    cases = [
        ("tiny_256x512", lambda: wl.weights(0, wl.tensor_id("tiny", 0), c0["N"], c0["K"]),
         lambda: wl.activations(0, wl.tensor_id("tiny", 1), 1, c0["K"]), 4),
        ("qwen7b_q_o_3584x3584", lambda: qwen("q_proj"), lambda: xh, 4),
        ("qwen7b_k_v_3584x512", lambda: qwen("k_proj"), lambda: xh, 4),
        ("qwen7b_gate_up_3584x18944", lambda: qwen("gate_proj"), lambda: xh, 4),
        ("qwen7b_down_18944x3584", lambda: qwen("down_proj"), lambda: xi, 4),
        ("qwen7b_qkv_fused_3584x4608",
         lambda: np.concatenate([qwen("q_proj"), qwen("k_proj"), qwen("v_proj")]), lambda: xh, 4),
        ("qwen7b_gate_up_fused_3584x37888",
         lambda: np.concatenate([qwen("gate_proj"), qwen("up_proj")]), lambda: xh, 4),
        ("lm_head_3584x152064", lambda: wl.weights(c3["seed"], wl.tensor_id("lm_head", 0), c3["N"], c3["K"]),
         lambda: wl.activations(c3["seed"], wl.tensor_id("lm_head", 1), 1, c3["K"]), 4),
        ("chatglm2_4096x27392", lambda: wl.weights(c2["seed"], wl.tensor_id("chatglm2", 0), c2["N"], c2["K"]),
         lambda: wl.activations(c2["seed"], wl.tensor_id("chatglm2", 1), 1, c2["K"], dtype=np.float16), 8),
    ]
    for name, mkW, mkX, bits in cases:
        progress("config " + name)
        W, X = mkW(), mkX()
        N, K = W.shape
        if bits == 4:
            t, R, tb = w4_config_times(qw, torch, W, X, pool, launches)
            b = bytes_w4a8(1, N, K)
        else:
            t, R, tb = w8_config_times(qw, torch, W, X, pool, launches)
            b = bytes_w8a16(1, N, K)
        line = {"op": "gemv_w4a8" if bits == 4 else "gemv_w8a16", "M": 1, "K": K, "N": N,
                "us": round(t, 3), "algo_bytes": b, "GB/s": round(b / t / 1e3, 1),
                "frac_of_peak": round(b / t / 1e3 / PEAK_HBM_GBS, 4),
                "bare_read_us": round(tb, 3), "frac_of_bare_read": round(tb / t, 4),
                "weight_copies_rotated": R}
        if with_oracle:
            if bits == 4:
                q, sc = oracle.quant_w4(W)
                run = {n: (lambda n=n: oracle.gemv_w4a8(X, q, sc, nthreads=n)) for n in (1, nt)}
            else:
                q, sc = oracle.quant_w8(W)
                run = {n: (lambda n=n: oracle.gemv_w8a16_ref64(X, q, sc, nthreads=n)) for n in (1, nt)}
            big = N * K > 200_000_000
            line["oracle_ms"] = {"1_thread": round(oracle_ms(run[1], 1 if big else 3), 3),
                                 "%d_threads" % nt: round(oracle_ms(run[nt], 3), 3)}
            del q, sc, run
        lines[name] = line
        del W
        torch.cuda.empty_cache()
    return lines


def chain_measurement(qw, wl, torch, replays):
    """Linear-layer time per token of the decode step: 28 layers of the seven Qwen-7B
    W4A8 linears plus the 3584 -> 152064 lm_head, captured in one HIP graph, unfused
    (197 launches) and with q|k|v and gate|up fused (113 launches).  Each layer streams
    its own copy of the packed weights."""
    from bit_weight_quantized_load_amd import chain

    seed = wl.QWEN7B_W4A8["seed"]
    layer = {}
    for name, K, N in wl.QWEN7B_LINEARS:
        W = wl.weights(seed, wl.tensor_id(name, 0), N, K, outlier_rows=True)
        layer[name] = qw.quantize_pack_w4(torch.from_numpy(W).cuda())
        del W
    c3 = wl.LMHEAD_W4A8
    W = wl.weights(c3["seed"], wl.tensor_id("lm_head", 0), c3["N"], c3["K"])
    lm = qw.quantize_pack_w4(torch.from_numpy(W).cuda())
    del W
    xh = torch.from_numpy(wl.activations(seed, wl.tensor_id("q_proj", 1), 1, wl.HIDDEN,
                                         outlier_channels=4)).cuda()
    xi = torch.from_numpy(wl.activations(seed, wl.tensor_id("down_proj", 1), 1, wl.INTERMEDIATE,
                                         outlier_channels=4)).cuda()
    out = {}
    for key, fused in (("unfused", False), ("fused_qkv_gate_up", True)):
        c = chain.DecodeChain(layer, lm, xh, xi, layers=wl.LAYERS, fused=fused)
        g = c.capture()
        t0 = time.perf_counter()
        while True:  # untimed replays, at least WARM_S seconds
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / replays
        b = c.bytes_per_token
        out[key] = {"launches_per_token": c.launches_per_token, "us_per_token": round(us, 2),
                    "tokens_per_s": round(1e6 / us, 1), "algo_bytes_per_token": b,
                    "GB/s": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
        del c, g
        torch.cuda.empty_cache()
    out["layers"] = wl.LAYERS
    out["replays"] = replays
    return out


def index_softmax_measurement(qw, torch, launches):
    """IndexSoftmax (the integer softmax of the IntAttention summary) on attention-like
    int32 logits: 8192 rows (2 heads x 4096 queries) of 4096 keys, d = 128, (b, c) =
    (5, 6.6); 4 B read and 1 B written per logit; input copies rotated past the cache."""
    rows, L, d = 8192, 4096, 128
    s_q, s_k = 0.02, 0.03
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    z = torch.randn((rows, L), generator=g, device="cuda") * 3.0
    A = torch.round(z * (d ** 0.5) / (s_q * s_k)).to(torch.int32)
    del z
    ci = qw.index_cint(6.6, d, s_q, s_k)
    R = max(2, math.ceil(ROTATE_BYTES / (A.numel() * 4)))
    copies = [A] + [A.clone() for _ in range(R - 1)]
    P = torch.empty((rows, L), dtype=torch.uint8, device="cuda")
    n = max(20, launches // 20)
    qw.index_softmax(A, ci, out=P)
    torch.cuda.synchronize()
    us = graph_us(torch, lambda i: qw.index_softmax(copies[i % R], ci, out=P), n)
    b = rows * L * 5
    del copies, A, P
    torch.cuda.empty_cache()
    return {"rows": rows, "L": L, "c_int": ci, "us": round(us, 2), "algo_bytes": b,
            "GB/s": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}


PEAK_MFMA_I8_TOPS = 5000.0   # dense int8 matrix cores
PEAK_MFMA_F16_TFLOPS = 2500.0  # dense f16 matrix cores


def skinny_sweep_measurement(qw, wl, torch, launches, c=None):
    """The skinny-GEMM sweep: gemv_w4a8 and gemv_w8a16 on their default paths for each M
    of the sweep, weight copies rotated past the cache; by default ChatGLM2's 4096 ->
    27392 linear (the GEMV kernels at M = 1, the matrix-core kernels above), or the
    given config (the long-K down projection: the long-K kernels up to 16 rows).
    Reports time, HBM bandwidth of the algorithmic bytes, and the rate against the dense
    matrix-core peak (int8 for W4A8, f16 for W8A16)."""
    c = wl.SKINNY if c is None else c
    K, N = c["K"], c["N"]
    W = torch.from_numpy(wl.weights(c["seed"], 1, N, K, outlier_rows=True)).cuda()
    Wq4, s4 = qw.quantize_pack_w4(W)
    Wq8, s8 = qw.quantize_pack_w8(W)
    del W
    R = max(2, math.ceil(ROTATE_BYTES / (Wq4.numel() + Wq8.numel())))
    copies = [(Wq4, s4, Wq8, s8)] + [(Wq4.clone(), s4.clone(), Wq8.clone(), s8.clone())
                                     for _ in range(R - 1)]
    n = max(R, 20)  # every rotated copy is read in each timed replay
    out = {"workload": c["workload"], "K": K, "N": N, "launches": n, "weight_copies_rotated": R,
           "timing": "median of 3 graph replays of %d launches after an untimed one" % n}

    def timed(fn):
        return graph_us(torch, fn, n)

    for M in c["Ms"]:
        progress("%s M=%d" % (c["workload"], M))
        X = torch.from_numpy(wl.activations(c["seed"], 2, M, K, outlier_channels=4)).cuda()
        X16 = X.half()
        Y4 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        Y8 = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ws4 = qw.make_workspace("w4a8", M, N, K)
        t4 = timed(lambda i: qw.gemv_w4a8(X, copies[i % R][0], copies[i % R][1], workspace=ws4, out=Y4))
        t8 = timed(lambda i: qw.gemv_w8a16(X16, copies[i % R][2], copies[i % R][3], out=Y8))
        row = {}
        for key, t, b, peak in (("w4a8", t4, bytes_w4a8(M, N, K), PEAK_MFMA_I8_TOPS),
                                ("w8a16", t8, bytes_w8a16(M, N, K), PEAK_MFMA_F16_TFLOPS)):
            tf = 2.0 * M * N * K / t / 1e6
            row[key] = {"us": round(t, 3), "algo_bytes": b, "GB/s": round(b / t / 1e3, 1),
                        "frac_of_hbm": round(b / t / 1e3 / PEAK_HBM_GBS, 4),
                        "T(FL)OP/s": round(tf, 2), "frac_of_mfma": round(tf / peak, 4)}
        out["M=%d" % M] = row
        del X, X16, Y4, Y8, ws4
    del copies, Wq4, s4, Wq8, s8
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the 28-layer decode-step chain measurement")
    ap.add_argument("--chain-replays", type=int, default=20)
    ap.add_argument("--no-skinny", action="store_true",
                    help="skip the skinny-GEMM sweeps (K = 4096, N = 27392, M = 1 .. 512; "
                         "K = 18944, N = 3584, M = 1 .. 16)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config M = 1 lines (each linear alone, beside a bare "
                         "read of its bytes and the oracle's time)")
    ap.add_argument("--no-index-softmax", action="store_true",
                    help="skip the IndexSoftmax measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run --steps device-to-device copies of BYTES bytes (a plain "
                         "copy kernel of known size, to calibrate HBM byte counters) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="(no GPU) write profiles/traffic_*.json from the counter CSVs of "
                         "four rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE on the copy "
                         "calibration, then FETCH_SIZE and WRITE_SIZE on this benchmark")
    ap.add_argument("--pmc-commands", default="",
                    help="with --write-traffic: the four commands, separated by ';;'")
    args = ap.parse_args()

    if args.write_traffic:
        cmds = [c.strip() for c in args.pmc_commands.split(";;") if c.strip()]
        write_traffic(*args.write_traffic, copy_bytes=args.copy_calibration or 268435456,
                      commands=cmds)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the GEMV needs no communication; "
              "sharding across GPUs is a design note, not built); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from __graft_entry__ import _ensure_built

    _ensure_built()
    import bit_weight_quantized_load_amd as qw
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration
        src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(8)]
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for i in range(args.steps):
            dst.copy_(src[i % 8])
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    c = wl.HEADLINE
    M, K, N = c["M"], c["K"], c["N"]
    b4, b8 = bytes_w4a8(M, N, K), bytes_w8a16(M, N, K)
    b_step = b4 + b8

    # synthetic inputs of the Qwen-7B gate/up projection: 1% outlier rows, 4 outlier channels
    W = wl.weights(1, wl.tensor_id("gate_proj", 0), N, K, outlier_rows=True)
    X = wl.activations(1, wl.tensor_id("gate_proj", 1), M, K, outlier_channels=4)
    X16 = X.astype(np.float16)
    Wd = torch.from_numpy(W).cuda()
    Wq4, s4 = qw.quantize_pack_w4(Wd)
    Wq8, s8 = qw.quantize_pack_w8(Wd)
    GROUP = 128
    Wq4g, s4g = qw.quantize_pack_w4g(Wd, GROUP)
    del Wd
    R = max(2, math.ceil(ROTATE_BYTES / (Wq4.numel() + Wq8.numel())))
    copies = [(Wq4, s4, Wq8, s8)] + [(Wq4.clone(), s4.clone(), Wq8.clone(), s8.clone())
                                     for _ in range(R - 1)]
    Xd = torch.from_numpy(X).cuda()
    X16d = torch.from_numpy(X16).cuda()
    Y4 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Y8 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws4 = qw.make_workspace("w4a8", M, N, K)
    ws8 = qw.make_workspace("w8a16", M, N, K)

    Rg = max(2, math.ceil(ROTATE_BYTES / (Wq4g.numel() + 4 * s4g.numel())))
    copies_g = [(Wq4g, s4g)] + [(Wq4g.clone(), s4g.clone()) for _ in range(Rg - 1)]
    # the INT4 page's ablations on the same shape: FP16 weights, and INT4 weights unpacked
    # to float against fp32 activations (the W4A8 packed copies)
    W16 = torch.from_numpy(W.astype(np.float16)).cuda()
    R16 = max(2, math.ceil(ROTATE_BYTES / (2 * W16.numel())))
    copies16 = [W16] + [W16.clone() for _ in range(R16 - 1)]

    def w4(i):
        w4q, sc4, _, _ = copies[i % R]
        qw.gemv_w4a8(Xd, w4q, sc4, workspace=ws4, out=Y4)

    def w4g(i):
        wq, sc = copies_g[i % Rg]
        qw.gemv_w4a8g(Xd, wq, sc, N, GROUP, out=Y4)

    def f16(i):
        qw.gemv_f16(X16d, copies16[i % R16], out=Y8)

    def w4f(i):
        w4q, sc4, _, _ = copies[i % R]
        qw.gemv_w4f32(Xd, w4q, sc4, out=Y4)

    def w8(i):
        _, _, w8q, sc8 = copies[i % R]
        qw.gemv_w8a16(X16d, w8q, sc8, workspace=ws8, out=Y8)

    def step(i):
        w4(i)
        w8(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The K timed steps are launched as one HIP graph (a single host call), so the
    # time is GPU time, not Python launch overhead.  Two more graphs of K launches of
    # one kernel each give the per-kernel average launch duration from HIP events.
    K_steps = args.steps

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K_steps):
                fn(i)
        # untimed replays (at least WARM_S seconds) outside the timed region
        t0 = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break
        return g

    progress("headline step")
    g_step = capture(step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_step.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g_step

    # per-kernel average launch time: a graph of max(K, copies) launches of one kernel,
    # median of 3 replays timed with HIP events after an untimed one
    n_k = max(K_steps, R, Rg, R16)
    t4 = graph_us(torch, w4, n_k)
    t8 = graph_us(torch, w8, n_k)
    t4g = graph_us(torch, w4g, n_k)
    b4g = bytes_w4a8g(M, N, K, GROUP)
    t16 = graph_us(torch, f16, n_k)
    t4f = graph_us(torch, w4f, n_k)
    b16 = 2 * N * K + 2 * M * K + 2 * M * N
    ms_per_step = wall * 1e3 / K_steps
    value = b_step / (ms_per_step * 1e-3) / 1e9
    # the bare streaming read of the same bytes, rotated the same way: the ceiling a
    # weight-streaming kernel of this size meets on this GPU
    pool = ReadPool(torch)
    tr4, rr4 = pool.time_us(qw, b4, n_k)
    tr8, rr8 = pool.time_us(qw, b8, n_k)

    def kline(t, b, **extra):
        d = {"us": round(t, 3), "algo_bytes": b, "GB/s": round(b / t / 1e3, 1),
             "frac_of_peak": round(b / t / 1e3 / PEAK_HBM_GBS, 4)}
        d.update(extra)
        return d

    kernels = {
        "gemv_w4a8": kline(t4, b4, frac_of_bare_read=round(tr4 / t4, 4)),
        "gemv_w8a16": kline(t8, b8, frac_of_bare_read=round(tr8 / t8, 4)),
        # plain streaming reads of the two GEMVs' algorithmic bytes (qw_stream_read)
        "bare_read_34MB": kline(tr4, b4, copies_rotated=rr4),
        "bare_read_68MB": kline(tr8, b8, copies_rotated=rr8),
        # the group-wise INT4 variant (one scale per row and 128 k) on the same shape:
        # context, not part of the step
        "gemv_w4a8g_g128": kline(t4g, b4g),
        # the page's ablations (context): FP16 GEMV, and weight-only INT4 unpacked to float
        "ablation_fp16_gemv": kline(t16, b16),
        "ablation_w4_float_unpack": kline(t4f, b4),
    }
    dom = "gemv_w8a16" if t8 >= t4 else "gemv_w4a8"
    ach = kernels[dom]["GB/s"]
    traffic = load_traffic(dom, c["workload"])
    roofline = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": dom}

    del copies, copies_g, copies16, W16
    torch.cuda.empty_cache()
    configs = None if args.no_configs else configs_measurement(
        qw, wl, torch, pool, K_steps, with_oracle=not args.no_cpu_baseline)
    del pool
    torch.cuda.empty_cache()
    progress("index softmax")
    isoft = None if args.no_index_softmax else index_softmax_measurement(qw, torch, K_steps)
    progress("skinny sweep")
    skinny = None if args.no_skinny else skinny_sweep_measurement(qw, wl, torch, K_steps)
    long_k = None if args.no_skinny else skinny_sweep_measurement(qw, wl, torch, K_steps, wl.LONG_K)
    chain_info = None
    if not args.no_chain:
        progress("decode chain")
        chain_info = chain_measurement(qw, wl, torch, args.chain_replays)

    cpu = None
    if not args.no_cpu_baseline:
        progress("oracle on the host")
        cpu = cpu_baseline(W, X, X16, args.cpu_seconds, b_step)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K_steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8xi8->i32 (W4A8), f16xf16->f32 (W8A16)", "data": "synthetic",
        "config": {"workload": c["workload"], "M": M, "K": K, "N": N,
                   "step": "gemv_w4a8 + gemv_w8a16", "weight_copies_rotated": R},
        "kernels": kernels, "roofline": roofline, "cpu_baseline": cpu,
        "configs": configs,
        "decode_chain": chain_info,
        "index_softmax": isoft,
        "skinny_sweep": skinny,
        "long_k_sweep": long_k,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
