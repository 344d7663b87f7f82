"""Benchmark of the ternary GEMV hot path at M = 1 on one MI355X.

Step (the `value` line): one pass of the hot path over the shapes the metric
names, [N, K] = [2560, 6912] (2B-4T down projection) and [8192, 28672]
(70B-class down projection), plus the transposed 70B-class shape
[28672, 8192]: for each, per-token int8 quantization of a bf16 activation
and the ternary GEMV with its fp32 rescale, in one launch (tq_quant_gemv;
bit-identical to tq_act_quant followed by tq_gemv, which is timed too).
`value` = packed weight bytes per step / step time (GB/s).

Inputs: seeded synthetic ternary weights (P(0) = 0.35), packed on the GPU
by tq_pack; bf16 N(0,1) activations.  Everything is resident in HBM before
timing starts.

Timing:
  * Each shape has a pool of distinct packed copies of at least 1 GiB, so
    the 256 MB Infinity Cache cannot serve repeats: step i uses copy
    i mod C of every pool (C = the pool's copy count).
  * Steps and kernel loops are captured in HIP graphs; a spin kernel queued
    before the start event keeps the host ahead, so HIP events on the
    launch stream measure GPU execution only.  The K timed steps are
    captured as ceil(K / 12) graphs of consecutive steps whose sizes differ
    by at most one (K = 20: two graphs of 10), so the fixed cost of a graph
    replay (about 5 us) is spread as in a decode graph of a layer stack;
    the time with one step per graph is reported too.
  * roofline: the dominant kernel (the fused [8192, 28672] launch) is timed
    as graphs of 96 back-to-back launches over its pool; algorithmic bytes
    per launch (packed weights + bf16 x + int8 x written + fp32 scale +
    fp32 y) / time per launch, against 8 TB/s.  Beside it, the measured
    read ceiling: tq_stream_read (16-byte non-temporal loads and nothing
    else) over the same pool (one 58.7 MB buffer per launch) and over one
    2 GiB buffer (the asymptotic rate, without the fixed cost of a launch).
  * per_shape: the step's shapes plus the 8B-class layers [14336, 4096] and
    [4096, 14336] and the 70B-class shards of an 8-way tensor-parallel split
    ([3584, 8192] gate/up, [8192, 3584] down), fused and int8 GEMV each, with
    the read ceiling at the same bytes per launch (tq_stream_read over the
    same pool) and each form's fraction of it.
  * rows: every hot-path row timed the same way -- act_quant, gemv, fused
    gate/up + relu^2 (2B-4T and 70B-class), the decode chain (30 2B-4T
    layers, graph-captured and, for comparison, launched eagerly; 8
    70B-class layers), the small-batch MFMA GEMM
    (M = 4, 16, 64), the absmean
    ternarizer, split-KV decode attention and the 30-layer decode-step chain
    (graph-captured).
  * cpu_baseline: the CPU oracle (plain C) on the same step, once on one
    thread and once on every host core the process may use (output rows
    split over threads), about 10 s each; `value` is the all-core rate.
Prints one JSON line on stdout; progress on stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("ternary GEMV weight GB/s + % of MI355X HBM peak at M=1 "
          "(2560x6912, 8192x28672)")
SHAPES = {"down_2b4t": (2560, 6912), "70b_down": (8192, 28672),
          "70b_up": (28672, 8192)}
# timed per shape beside the step: 8B-class layers, 70B-class TP=8 shards
EXTRA_SHAPES = {"8b_up": (14336, 4096), "8b_down": (4096, 14336),
                "70b_tp8_gate_up": (3584, 8192), "70b_tp8_down": (8192, 3584)}
DOMINANT = "70b_down"
HBM_PEAK_GBS = 8000.0
INT8_MFMA_PEAK_TOPS = 5000.0
POOL_BYTES_MIN = 1 << 30
STEP_COPIES = 12        # steps per graph
BIG_READ_BYTES = 2 << 30
SPIN = 20_000_000
COUNTER_FILE = os.path.join(ROOT, "profiles", "tq_quant_gemv_8192x28672_counters.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "bench_kernel_trace.txt")
KERNEL_SOURCES = ("bit_gemv_tq_amd/csrc/tq_gemv_reg.h",
                  "bit_gemv_tq_amd/csrc/tq_gemv.hip",
                  "bit_gemv_tq_amd/csrc/tq_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(N, K):
    return N * K // 4


def algo_bytes(N, K, M=1):
    # packed weights + int8 activations + fp32 x_scale + fp32 outputs
    return N * K // 4 + M * K + 4 * M + 4 * M * N


def algo_bytes_fused(N, K):
    # packed weights + bf16 row read + int8 row and scale written + fp32 y
    return N * K // 4 + 2 * K + K + 4 + 4 * N


def graph_sizes(steps):
    """Steps per graph for `steps` consecutive timed steps: ceil(steps /
    STEP_COPIES) graphs whose sizes differ by at most one, so no step is
    charged a graph of its own (a graph replay has a fixed cost of about
    5 us on this part, which a graph of one 3-kernel step would charge to
    every step, while a decode graph holds a whole layer stack)."""
    n = -(-steps // STEP_COPIES)
    return [steps // n + (1 if g < steps % n else 0) for g in range(n)]


def code_only(text):
    """Source text without // comments and blank lines: a comment edit does
    not change the kernel the counters were taken on."""
    lines = (re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l)


def kernel_source_hash(read=None):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def read_profile(path):
    """key: value fields of a committed rocprofv3 summary, or None unless it
    was taken on the current kernel source."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return fields


def read_traffic():
    """HBM bytes per dominant-kernel launch from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    f = read_profile(COUNTER_FILE)
    try:
        return float(f["hbm_bytes_per_launch"]) if f else None
    except (KeyError, ValueError):
        return None


def read_trace():
    """The dominant kernel's rocprofv3 kernel-trace average and median (us),
    if the committed trace was taken on the current kernel source."""
    f = read_profile(TRACE_FILE)
    try:
        return (float(f["dominant_trace_avg_us"]),
                float(f["dominant_trace_median_us"])) if f else None
    except (KeyError, ValueError):
        return None


def trace_fields(tr, nbytes):
    """The committed kernel-trace figures of the dominant kernel (when taken
    on the current kernel source), with the fraction of peak they give."""
    if tr is None:
        return None
    avg, med = tr
    return {"avg_us": avg, "median_us": med,
            "frac_from_avg": round(nbytes / avg / 1e3 / HBM_PEAK_GBS, 4),
            "frac_from_median": round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4),
            "file": os.path.relpath(TRACE_FILE, ROOT)}


def cpu_info():
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count(), usable


def cpu_baseline(budget_s=10.0, max_threads=16):
    """The CPU oracle on the same step: one thread, then all usable cores
    (at most `max_threads`: the host share of one GPU) with each GEMV's
    packed rows split into contiguous slices, one oracle call per slice on
    its own thread (the oracle is plain C called through ctypes, which
    releases the GIL, so the calls run in parallel).  The oracle itself is
    unchanged; each output row is still summed by one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import workloads
    packed, xbits = {}, {}
    for t, (name, (N, K)) in enumerate(SHAPES.items()):
        codes = workloads.ternary_codes(N, K, seed=workloads.seed_for(5, t))
        packed[name] = oracle.pack(codes)
        del codes
        xbits[name] = workloads.activations_bf16(1, K, seed=workloads.seed_for(5, 10 + t))
    s_w = np.float32(0.02)
    model, ncpu, usable = cpu_info()
    threads = max(1, min(usable, max_threads))
    pool = ThreadPoolExecutor(threads)

    def gemv_split(name, N, q, s, nt):
        n4 = N // 4
        cuts = [n4 * i // nt for i in range(nt + 1)]
        jobs = [pool.submit(oracle.gemv, packed[name][a:b], s_w, q, s, 4 * (b - a))
                for a, b in zip(cuts, cuts[1:]) if b > a]
        return [j.result() for j in jobs]

    step_bytes = sum(weight_bytes(*s) for s in SHAPES.values())

    def run(nt, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for name, (N, K) in SHAPES.items():
                q, s = oracle.act_quant(xbits[name], "bf16")
                if nt == 1:
                    oracle.gemv(packed[name], s_w, q, s, N)
                else:
                    gemv_split(name, N, q, s, nt)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 80:
                return reps, el

    def median_of(nt, runs=5):
        """Median weight GB/s of `runs` timed runs (the budget split
        between them), with the runs themselves."""
        rs = [run(nt, budget_s / runs) for _ in range(runs)]
        rates = sorted(step_bytes * r / e / 1e9 for r, e in rs)
        return rates[len(rates) // 2], rs

    one, rs1 = median_of(1)
    alln, rsn = median_of(threads)
    pool.shutdown()
    fmt = lambda rs: ", ".join(f"{r} in {e:.2f} s" for r, e in rs)
    return {"value": round(alln, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"median of 5 runs of full steps (all three shapes, act_quant + "
                       f"GEMV) on {threads} threads, output rows split over threads "
                       f"({fmt(rsn)}); one thread: median of 5 ({fmt(rs1)})"),
            "one_thread_value": round(one, 4),
            "host": {"cpu_model": model, "nproc": ncpu, "usable_cores": usable}}


def cpu_rows(budget_s=3.0):
    """The CPU oracle on a bounded sample of each hot-path row (one thread):
    per row, repeated calls for about `budget_s` seconds; weight GB/s (or
    tokens/s for the chain) of the oracle as it stands."""
    import numpy as np

    import oracle
    import workloads

    def timed(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return reps, el

    out = {}
    H, I = workloads.HIDDEN, workloads.INTERMEDIATE
    # a1 act-quant, M = 1, K = 6912
    xb = workloads.activations_bf16(1, I, seed=501)
    reps, el = timed(lambda: oracle.act_quant(xb, "bf16"))
    out["act_quant_M1_K6912"] = {"us_per_call": round(el / reps * 1e6, 1),
                                 "sample": f"{reps} calls"}
    # a4 gate/up + relu^2 M = 1 [6912, 2560] x 2
    pg = oracle.pack(workloads.ternary_codes(I, H, seed=502))
    pu = oracle.pack(workloads.ternary_codes(I, H, seed=503))
    q, sx = oracle.act_quant(workloads.activations_bf16(1, H, seed=504), "bf16")
    reps, el = timed(lambda: oracle.gate_up_relu2(pg, 0.024, pu, 0.025, q, sx, I))
    out["gate_up_relu2_M1_6912x2560"] = {
        "weight_GBs": round(2 * weight_bytes(I, H) * reps / el / 1e9, 4),
        "sample": f"{reps} calls"}
    # a5 small-batch GEMM, M = 16, [2560, 6912]
    pd = oracle.pack(workloads.ternary_codes(H, I, seed=505))
    q16, s16 = oracle.act_quant(workloads.activations_bf16(16, I, seed=506), "bf16")
    reps, el = timed(lambda: oracle.gemv(pd, 0.02, q16, s16, H))
    out["gemm_small_M16_2560x6912"] = {
        "weight_GBs": round(weight_bytes(H, I) * reps / el / 1e9, 4),
        "int8_GOPS": round(2 * 16 * H * I * reps / el / 1e9, 3),
        "sample": f"{reps} calls"}
    # a6 decode chain: 2 layers of the 30 (per-layer cost x 30 = per token)
    layers = []
    for l in range(2):
        layer = {}
        for name, (N, K) in workloads.LAYER_2B4T.items():
            t = workloads.TENSOR_INDEX[name]
            layer[name] = (oracle.pack(workloads.ternary_codes(
                N, K, seed=workloads.seed_for(2, t, l))), workloads.tensor_scale(t), N)
        layers.append(layer)
    h0 = workloads.activations_bf16(1, H, seed=507, outliers=True)
    reps, el = timed(lambda: oracle.decode_chain(layers, h0))
    per_layer = el / reps / 2
    out["decode_chain_30x2b4t"] = {
        "us_per_token": round(per_layer * workloads.CHAIN_LAYERS * 1e6, 1),
        "tokens_per_s": round(1 / (per_layer * workloads.CHAIN_LAYERS), 3),
        "sample": f"{reps} passes over 2 layers, scaled to 30"}
    # next-1 absmean ternarizer on [2560, 6912] bf16 weights
    wb = workloads.weights_bf16(H, I, seed=508)
    reps, el = timed(lambda: oracle.ternarize(wb))
    out["ternarize_2560x6912"] = {
        "bf16_weight_GBs": round(2 * H * I * reps / el / 1e9, 4),
        "sample": f"{reps} calls"}
    # next-4 decode attention, 2B-4T heads, L = 2048
    rng = np.random.default_rng(509)
    qa = rng.standard_normal((20, 128)).astype(np.float32)
    kb = (rng.standard_normal((2048, 5, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (rng.standard_normal((2048, 5, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    reps, el = timed(lambda: oracle.attn_decode(qa, kb, vb, np.float32(128 ** -0.5)))
    out["attn_decode_L2048"] = {"us_per_call": round(el / reps * 1e6, 1),
                                "sample": f"{reps} calls"}
    out["cores"] = 1
    return out


class Timer:
    """Graph-captured launch sequences timed with HIP events."""

    def __init__(self, torch):
        self.torch = torch

    def graph(self, fn):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_sequence(self, graphs, steps):
        """ms per step: `graphs` (together exactly `steps` steps) replayed
        once each, in order."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN)
        e0.record()
        for g in graphs:
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_graphs(self, graphs, reps):
        """ms per replay, cycling through `graphs` for `reps` replays."""
        torch = self.torch
        for g in graphs[:2]:
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN)
        e0.record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-row table (gate/up, GEMM, chain)")
    ap.add_argument("--kernel-reps", type=int, default=96,
                    help="launches per graph in the per-kernel loops")
    ap.add_argument("--counters", action="store_true",
                    help="only run a 256 MiB calibration copy, the dominant kernel, "
                         "the int8 GEMV and the five-per-byte GEMV at its shape, 8 "
                         "launches each (for rocprofv3 --pmc runs), then exit")
    ap.add_argument("--counters-gemm", action="store_true",
                    help="only run the small-batch GEMM at each benchmarked "
                         "(M, N, K), 8 launches each (for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_gemv_tq_amd as tq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timer = Timer(torch)
    s_w = np.float32(0.02)

    if args.counters:
        counters_run(torch, tq, workloads, dev)
        return
    if args.counters_gemm:
        gemm_counters_run(torch, tq, workloads, dev)
        return

    # ---------------------------------------------------------------- pools
    def make_pool(N, K, copies, seed0):
        out = []
        for c in range(copies):
            w = workloads.ternary_codes_torch(N, K, seed=seed0 + c, device=dev)
            out.append(tq.tq_pack(w))
            del w
        return out

    ALL = dict(SHAPES, **EXTRA_SHAPES)
    pools = {}
    for t, (name, (N, K)) in enumerate(ALL.items()):
        copies = max(STEP_COPIES, -(-POOL_BYTES_MIN // weight_bytes(N, K)))
        log(f"pool {name}: {copies} copies x {weight_bytes(N, K) / 1e6:.1f} MB")
        pools[name] = make_pool(N, K, copies, workloads.seed_for(4, t) * 1000 + 7)
    torch.cuda.synchronize()
    x, xq, xs, y = {}, {}, {}, {}
    for t, (name, (N, K)) in enumerate(ALL.items()):
        xb = workloads.activations_bf16(1, K, seed=workloads.seed_for(4, 20 + t))
        x[name] = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)[0]
        xq[name] = torch.empty(K, dtype=torch.int8, device=dev)
        xs[name] = torch.empty(1, dtype=torch.float32, device=dev)
        y[name] = torch.empty(N, dtype=torch.float32, device=dev)

    def step(i):  # step i reads copy i mod C of every pool
        for name in SHAPES:
            P = pools[name]
            tq.tq_quant_gemv(x[name], P[i % len(P)], s_w, y[name],
                             xq=xq[name], x_scale=xs[name])

    def step_unfused(i):
        for name in SHAPES:
            P = pools[name]
            tq.tq_act_quant(x[name], xq[name], xs[name])
            tq.tq_gemv(P[i % len(P)], s_w, xq[name], xs[name], y[name])

    def steps_of(fn, i0, n):
        def run():
            for i in range(i0, i0 + n):
                fn(i)
        return run

    def step_graphs(fn, steps):
        """Graphs for steps 0 .. steps-1, consecutive steps per graph as
        graph_sizes gives them, each with its size."""
        out, i0 = [], 0
        for n in graph_sizes(steps):
            out.append((timer.graph(steps_of(fn, i0, n)), n))
            i0 += n
        return out

    def warm(graphs, warmup):
        done = 0
        for g, n in graphs:
            if done >= warmup:
                break
            g.replay()
            done += n
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- step
    log("capturing step graphs")
    graphs = step_graphs(step, args.steps)
    warm(graphs, args.warmup)
    wall0 = time.perf_counter()
    ms_step = timer.time_sequence([g for g, _ in graphs], args.steps)
    wall = time.perf_counter() - wall0
    step_wbytes = sum(weight_bytes(*s) for s in SHAPES.values())
    value = step_wbytes / (ms_step * 1e-3) / 1e9
    log(f"step: {ms_step * 1e3:.2f} us -> {value:.0f} GB/s")
    del graphs
    singles = [timer.graph(steps_of(step, i, 1)) for i in range(STEP_COPIES)]
    ms_step_1 = timer.time_graphs(singles, args.steps)
    log(f"step, one step per graph: {ms_step_1 * 1e3:.2f} us")
    del singles
    graphs_u = step_graphs(step_unfused, args.steps)
    warm(graphs_u, STEP_COPIES)
    ms_step_u = timer.time_sequence([g for g, _ in graphs_u], args.steps)
    log(f"unfused step (act_quant + gemv launches): {ms_step_u * 1e3:.2f} us")
    del graphs_u

    # ------------------------------------------------- per-kernel loops
    R = args.kernel_reps

    # RMSNorm weights for the norm-fused variant (next-2: the sub-layer norm
    # in the GEMV prologue), bf16 like the activations
    gam = {name: (1.0 + 0.1 * torch.randn(K, device=dev)).to(torch.bfloat16)
           for name, (N, K) in SHAPES.items()}

    def gemv_loop(name, start, mode):
        P = pools[name]
        for r in range(R):
            if mode == "quant_gemv":
                tq.tq_quant_gemv(x[name], P[(start + r) % len(P)], s_w, y[name],
                                 xq=xq[name], x_scale=xs[name])
            elif mode == "rmsnorm_quant_gemv":
                tq.tq_rmsnorm_quant_gemv(x[name], gam[name], P[(start + r) % len(P)],
                                         s_w, eps=1e-5, y=y[name], xq=xq[name],
                                         x_scale=xs[name])
            else:
                tq.tq_gemv(P[(start + r) % len(P)], s_w, xq[name], xs[name], y[name])

    sink = torch.zeros(4096, 4, dtype=torch.int32, device=dev)

    def read_pool_loop(name, start):
        P = pools[name]
        for r in range(R):
            tq.tq_stream_read(P[(start + r) % len(P)], sink)

    per_shape = {}
    for name, (N, K) in ALL.items():
        tq.tq_act_quant(x[name], xq[name], xs[name])
        nP = len(pools[name])
        row = {"N": N, "K": K, "pool_copies": nP}
        modes = ("quant_gemv", "gemv") + (("rmsnorm_quant_gemv",) if name in SHAPES else ())
        for mode in modes:
            fused = mode != "gemv"
            gs = [timer.graph(lambda name=name, s=s, m=mode: gemv_loop(name, s, m))
                  for s in range(0, nP, max(1, nP // 4))][:4]
            us = timer.time_graphs(gs, 8) * 1e3 / R
            # the norm-fused form also reads K gamma values (bf16)
            ab = (algo_bytes_fused(N, K) + (2 * K if mode == "rmsnorm_quant_gemv" else 0)
                  if fused else algo_bytes(N, K))
            row[mode] = {
                "us_per_launch": round(us, 3),
                "weight_GBs": round(weight_bytes(N, K) / us / 1e3, 1),
                "pct_hbm_peak": round(100 * weight_bytes(N, K) / us / 1e3 / HBM_PEAK_GBS, 1),
                "algo_GBs": round(ab / us / 1e3, 1)}
            del gs
        # the read ceiling at this shape: tq_stream_read over the same pool,
        # one packed matrix per launch (the same bytes and launch count)
        gs = [timer.graph(lambda name=name, s=s: read_pool_loop(name, s))
              for s in range(0, nP, max(1, nP // 4))][:4]
        rus = timer.time_graphs(gs, 8) * 1e3 / R
        del gs
        row["read_ceiling_us"] = round(rus, 3)
        for mode in modes:
            row[mode]["frac_of_read_ceiling"] = round(rus / row[mode]["us_per_launch"], 3)
        per_shape[name] = row
        log(f"{name}: {row}")

    dN, dK = SHAPES[DOMINANT]
    dom_us = per_shape[DOMINANT]["quant_gemv"]["us_per_launch"]
    achieved = algo_bytes_fused(dN, dK) / dom_us / 1e3

    # the measured read ceiling: a read-only kernel (tq_stream_read, the
    # GEMV's 16-byte non-temporal access and nothing else) over the same pool
    read_us = per_shape[DOMINANT]["read_ceiling_us"]
    read_gbs = weight_bytes(dN, dK) / read_us / 1e3
    ceiling = {"us_per_launch": round(read_us, 3), "GBs": round(read_gbs, 1),
               "pct_hbm_peak": round(100 * read_gbs / HBM_PEAK_GBS, 1),
               "bytes": weight_bytes(dN, dK)}
    log(f"read ceiling over the {DOMINANT} pool: {ceiling}")
    # ... and over one 2 GiB buffer per launch: the asymptotic read rate,
    # where the fixed cost of a launch (dispatch, first-load latency, drain)
    # no longer counts
    big = torch.ones(BIG_READ_BYTES, dtype=torch.uint8, device=dev)

    def big_loop():
        for _ in range(8):
            tq.tq_stream_read(big, sink)
    g = timer.graph(big_loop)
    big_us = timer.time_graphs([g], 2) * 1e3 / 8
    del g, big
    ceiling["large_buffer"] = {"us_per_launch": round(big_us, 2), "bytes": BIG_READ_BYTES,
                               "GBs": round(BIG_READ_BYTES / big_us / 1e3, 1),
                               "pct_hbm_peak": round(100 * BIG_READ_BYTES / big_us / 1e3
                                                     / HBM_PEAK_GBS, 1)}
    log(f"read ceiling over one 2 GiB buffer: {ceiling['large_buffer']}")

    rows = {}
    if not args.no_rows:
        rows = measure_rows(torch, tq, workloads, timer, dev, R, per_shape)

    cpu = None if args.no_cpu else cpu_baseline()
    if cpu is not None and not args.no_rows:
        log("cpu oracle rows")
        cpu["rows"] = cpu_rows()
        log(f"cpu rows: {cpu['rows']}")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": ("ternary GEMV at M=1, [N,K] = [2560,6912] (2B-4T down), "
                         "[8192,28672] and [28672,8192] (70B-class, both "
                         "orientations); per shape act_quant(bf16) + gemv per step"),
            "weight_bytes_per_step": step_wbytes,
            "pool_copies_per_shape": {k: len(pools[k]) for k in SHAPES},
            "pool_bytes_min": POOL_BYTES_MIN,
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
            "steps_per_graph": graph_sizes(args.steps),
            "ms_per_step_one_step_per_graph": round(ms_step_1, 5),
            "unfused_ms_per_step": round(ms_step_u, 5),
            "read_ceiling": ceiling,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"gemv_reg_kernel (bf16 prologue), tq_quant_gemv [N,K]=[{dN},{dK}]",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(),
            "us_per_launch": dom_us,
            "time_source": ("live: HIP events around graphs of 96 back-to-back "
                            "launches cycling the 1 GiB pool, divided by the launch count"),
            "trace": trace_fields(read_trace(), algo_bytes_fused(dN, dK)),
            "bytes_per_launch": algo_bytes_fused(dN, dK),
            "read_ceiling_GBs": round(read_gbs, 1),
            "frac_of_read_ceiling": round(achieved / read_gbs, 4),
        },
        "per_shape": per_shape,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def counters_run(torch, tq, workloads, dev):
    """Dispatches for the HBM-traffic and instruction counters: a plain
    device-to-device copy of 256 MiB (calibration: its FETCH_SIZE and
    WRITE_SIZE should each read 256 MiB), then the dominant GEMV over 4
    distinct weight copies, the int8 GEMV on them, and the five-per-byte
    GEMV at the same shape."""
    import numpy as np
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    N, K = SHAPES[DOMINANT]
    P = []
    for c in range(4):
        w = workloads.ternary_codes_torch(N, K, seed=4242 + c, device=dev)
        P.append(tq.tq_pack(w))
        del w
    xb = workloads.activations_bf16(1, K, seed=4243)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)[0]
    q = torch.empty(K, dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    yy = torch.empty(N, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for r in range(8):
        tq.tq_quant_gemv(xt, P[r % 4], 0.02, yy, xq=q, x_scale=s)
    torch.cuda.synchronize()
    # the int8 GEMV on the same weights, then the five-per-byte GEMV on the
    # same shape (four distinct copies each)
    for r in range(8):
        tq.tq_gemv(P[r % 4], 0.02, q, s, yy)
    torch.cuda.synchronize()
    del P
    P3 = []
    for c in range(4):
        w = workloads.ternary_codes_torch(N, K, seed=4342 + c, device=dev)
        P3.append(tq.tq_pack3(w))
        del w
    torch.cuda.synchronize()
    for r in range(8):
        tq.tq_gemv3(P3[r % 4], 0.02, q, s, N, yy)
    torch.cuda.synchronize()
    log("counters run done")


def gemm_counters_run(torch, tq, workloads, dev):
    """Dispatches for the small-batch GEMM counters (MFMA operations and
    busy cycles, fetched bytes): a 256 MiB calibration copy, then for each
    benchmarked shape and M, 8 launches over 4 distinct weight copies."""
    import numpy as np
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for (N, K) in workloads.GEMM_SMALL_SHAPES:
        P = []
        for c in range(4):
            w = workloads.ternary_codes_torch(N, K, seed=5252 + c, device=dev)
            P.append(tq.tq_pack(w))
            del w
        for M in workloads.GEMM_SMALL_M:
            xb = workloads.activations_bf16(M, K, seed=95 + M)
            xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(M, K)
            q, s = tq.tq_act_quant(xt)
            yy = torch.empty(M, N, dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            log(f"gemm counters M={M} N={N} K={K}")
            for r in range(8):
                tq.tq_gemm_small(P[r % 4], 0.02, q, s, yy)
            torch.cuda.synchronize()
        del P
    log("gemm counters run done")


def measure_rows(torch, tq, workloads, timer, dev, R, per_shape):
    """Every hot-path row, graph-timed over cache-defeating pools."""
    import numpy as np
    from bit_gemv_tq_amd.chain import DecodeChain, Layer

    rows = {}

    def pool_of(N, K, min_bytes, seed0):
        copies = max(4, -(-min_bytes // weight_bytes(N, K)))
        out = []
        for c in range(copies):
            w = workloads.ternary_codes_torch(N, K, seed=seed0 + c, device=dev)
            out.append(tq.tq_pack(w))
            del w
        return out

    def loop_us(fn, nP, reps=8):
        gs = [timer.graph(lambda s=s: fn(s)) for s in range(0, nP, max(1, nP // 4))][:4]
        return timer.time_graphs(gs, reps) * 1e3 / R

    # a1: act_quant on bf16 rows (input cache-resident: it is reused)
    aq = {}  # us per launch; bytes 2K in + K + 4 out (latency bound)
    for K in (2560, 6912, 8192, 28672):
        xb = workloads.activations_bf16(1, K, seed=K)
        xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        q = torch.empty(K, dtype=torch.int8, device=dev)
        s = torch.empty(1, dtype=torch.float32, device=dev)

        def f(_, xt=xt, q=q, s=s):
            for _r in range(R):
                tq.tq_act_quant(xt, q, s)
        aq[K] = round(loop_us(f, 1), 3)
    rows["act_quant_us_per_launch_M1"] = aq
    log(f"act_quant: {aq}")

    # a2/a3 at the 2B-4T q_proj shape [2560, 2560] (the single-GEMV case)
    N, K = workloads.HIDDEN, workloads.HIDDEN
    P = pool_of(N, K, 640 << 20, 90000)
    xb = workloads.activations_bf16(1, K, seed=90)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    q, s = tq.tq_act_quant(xt)
    yq = torch.empty(N, dtype=torch.float32, device=dev)

    def fq(st):
        for r in range(R):
            tq.tq_gemv(P[(st + r) % len(P)], 0.02, q, s, yq)
    us = loop_us(fq, len(P))
    rows["gemv_q_proj_2560x2560"] = {
        "us_per_launch": round(us, 3),
        "weight_GBs": round(weight_bytes(N, K) / us / 1e3, 1),
        "pct_hbm_peak": round(100 * algo_bytes(N, K) / us / 1e3 / HBM_PEAK_GBS, 1)}
    log(f"gemv q_proj: {rows['gemv_q_proj_2560x2560']}")
    del P

    # next-3: the five-weights-per-byte layout (tq_gemv3) at the metric's
    # shapes, beside the two-bit int8 GEMV timed above
    g3 = {}
    for name, (N, K) in SHAPES.items():
        n5 = (N + 4) // 5
        b3 = n5 * K
        copies = max(4, -(-(640 << 20) // b3))
        P3 = []
        for c in range(copies):
            w = workloads.ternary_codes_torch(N, K, seed=96000 + c, device=dev)
            P3.append(tq.tq_pack3(w))
            del w
        xb = workloads.activations_bf16(1, K, seed=97)
        xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        q, s = tq.tq_act_quant(xt)
        y3 = torch.empty(N, dtype=torch.float32, device=dev)

        def f3(st, P3=P3, q=q, s=s, y3=y3, N=N):
            for r in range(R):
                tq.tq_gemv3(P3[(st + r) % len(P3)], 0.02, q[0], s, N, y3)
        us = loop_us(f3, len(P3))
        two_bit = per_shape[name]["gemv"]["us_per_launch"]
        g3[name] = {
            "us_per_launch": round(us, 3),
            "packed_bytes": b3,
            "packed_GBs": round(b3 / us / 1e3, 1),
            "pct_hbm_peak": round(100 * (b3 + K + 4 + 4 * N) / us / 1e3 / HBM_PEAK_GBS, 1),
            "tweights_per_s": round(N * K / us / 1e6, 2),
            "speedup_vs_2bit_gemv": round(two_bit / us, 3)}
        log(f"gemv3 {name}: {g3[name]}")
        del P3
    rows["gemv3_five_per_byte"] = g3

    # grouped q/k/v (one launch for the three projections that share x),
    # 2B-4T and 70B-class, against one concatenated matrix of the same bytes
    grp = {}
    for tag, Ns, K in (("2b4t_qkv", (2560, 640, 640), 2560),
                       ("70b_qkv", (8192, 1024, 1024), 8192)):
        P = [pool_of(N, K, (512 << 20) if N > 2048 else (128 << 20), 81000 + 1000 * c)
             for c, N in enumerate(Ns)]
        Cc = pool_of(sum(Ns), K, 1 << 30, 85000)
        xb = workloads.activations_bf16(1, K, seed=98)
        xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)[0]
        ys = [torch.empty(N, dtype=torch.float32, device=dev) for N in Ns]
        yc = torch.empty(sum(Ns), dtype=torch.float32, device=dev)
        xq1 = torch.empty(K, dtype=torch.int8, device=dev)
        xs1 = torch.empty(1, dtype=torch.float32, device=dev)
        nP = min(len(p) for p in P)

        def fgrp(st, P=P, xt=xt, ys=ys, xq1=xq1, xs1=xs1, nP=nP):
            for r in range(R):
                i = (st + r) % nP
                tq.tq_quant_gemv_group(xt, [p[i] for p in P], [0.02, 0.021, 0.022], ys,
                                       xq=xq1, x_scale=xs1)

        def fcat(st, Cc=Cc, xt=xt, yc=yc, xq1=xq1, xs1=xs1):
            for r in range(R):
                tq.tq_quant_gemv(xt, Cc[(st + r) % len(Cc)], 0.02, yc, xq=xq1, x_scale=xs1)
        us_g = loop_us(fgrp, nP)
        us_c = loop_us(fcat, len(Cc))
        wb = sum(weight_bytes(N, K) for N in Ns)
        grp[tag] = {"Ns": list(Ns), "K": K, "weight_bytes": wb,
                    "grouped_us": round(us_g, 3),
                    "grouped_weight_GBs": round(wb / us_g / 1e3, 1),
                    "one_matrix_us": round(us_c, 3)}
        log(f"grouped {tag}: {grp[tag]}")
        del P, Cc
    rows["quant_gemv_group_qkv"] = grp

    # a4: fused gate/up + relu^2, M = 1 (2B-4T MLP)
    N, K = workloads.INTERMEDIATE, workloads.HIDDEN
    pg = pool_of(N, K, 320 << 20, 91000)
    pu = pool_of(N, K, 320 << 20, 92000)
    xb = workloads.activations_bf16(1, K, seed=93)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    q, s = tq.tq_act_quant(xt)
    h = torch.empty(N, dtype=torch.float32, device=dev)

    def fg(st):
        for r in range(R):
            i = (st + r) % len(pg)
            tq.tq_gate_up_relu2(pg[i], 0.024, pu[i], 0.025, q, s, h)
    us = loop_us(fg, len(pg))
    rows["gate_up_relu2_M1_6912x2560"] = {
        "us_per_launch": round(us, 3),
        "weight_GBs": round(2 * weight_bytes(N, K) / us / 1e3, 1),
        "pct_hbm_peak": round(100 * (2 * weight_bytes(N, K) + K + 4 + 4 * N)
                              / us / 1e3 / HBM_PEAK_GBS, 1)}
    log(f"gate_up: {rows['gate_up_relu2_M1_6912x2560']}")
    del pg, pu

    # a4 at the 70B-class MLP: gate and up [28672, 8192] each, 117 MB of
    # weights per launch (the largest single hot-path launch), int8 row and
    # fused bf16 quantization, beside the read ceiling at the same bytes
    N, K = 28672, 8192
    pg = pool_of(N, K, 1 << 30, 93000)
    pu = pool_of(N, K, 1 << 30, 93500)
    xb = workloads.activations_bf16(1, K, seed=94)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    q, s = tq.tq_act_quant(xt)
    xq1 = torch.empty(K, dtype=torch.int8, device=dev)
    xs1 = torch.empty(1, dtype=torch.float32, device=dev)
    h = torch.empty(N, dtype=torch.float32, device=dev)
    wb2 = 2 * weight_bytes(N, K)

    def fg70(st):
        for r in range(R):
            i = (st + r) % len(pg)
            tq.tq_gate_up_relu2(pg[i], 0.024, pu[i], 0.025, q, s, h)

    def fq70(st):
        for r in range(R):
            i = (st + r) % len(pg)
            tq.tq_quant_gate_up_relu2(xt[0], pg[i], 0.024, pu[i], 0.025, h, xq=xq1,
                                      x_scale=xs1)
    us_i8 = loop_us(fg70, len(pg))
    us_fq = loop_us(fq70, len(pg))
    del pu
    # one buffer of both matrices' bytes per launch, 12 distinct buffers
    cat = [torch.empty(wb2, dtype=torch.uint8, device=dev) for _ in range(12)]
    for c in cat:
        c.random_(0, 255)
    sink = torch.zeros(4096, 4, dtype=torch.int32, device=dev)

    def fr70(st):
        for r in range(R):
            tq.tq_stream_read(cat[(st + r) % len(cat)], sink)
    us_rd = loop_us(fr70, len(cat))
    del pg, cat
    rows["gate_up_relu2_M1_70b_28672x8192"] = {
        "weight_bytes": wb2,
        "int8": {"us_per_launch": round(us_i8, 3),
                 "weight_GBs": round(wb2 / us_i8 / 1e3, 1),
                 "pct_hbm_peak": round(100 * wb2 / us_i8 / 1e3 / HBM_PEAK_GBS, 1),
                 "frac_of_read_ceiling": round(us_rd / us_i8, 3)},
        "quant_fused": {"us_per_launch": round(us_fq, 3),
                        "weight_GBs": round(wb2 / us_fq / 1e3, 1),
                        "pct_hbm_peak": round(100 * wb2 / us_fq / 1e3 / HBM_PEAK_GBS, 1),
                        "frac_of_read_ceiling": round(us_rd / us_fq, 3)},
        "read_ceiling_us": round(us_rd, 3),
        "read_ceiling_pct_hbm_peak": round(100 * wb2 / us_rd / 1e3 / HBM_PEAK_GBS, 1)}
    log(f"gate_up 70b: {rows['gate_up_relu2_M1_70b_28672x8192']}")

    # a5: small-batch GEMM on the int8 matrix cores
    gemm, gate = {}, {}
    for (N, K) in workloads.GEMM_SMALL_SHAPES:
        P = pool_of(N, K, 640 << 20, 94000 + N)
        for M in workloads.GEMM_SMALL_M:
            xb = workloads.activations_bf16(M, K, seed=95 + M)
            xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(M, K)
            q, s = tq.tq_act_quant(xt)
            yy = torch.empty(M, N, dtype=torch.float32, device=dev)

            def fm(st, P=P, q=q, s=s, yy=yy):
                for r in range(R):
                    tq.tq_gemm_small(P[(st + r) % len(P)], 0.02, q, s, yy)
            us = loop_us(fm, len(P))
            ops = 2.0 * M * N * K
            gemm[f"M{M}_{N}x{K}"] = {
                "us_per_launch": round(us, 3),
                "weight_GBs": round(weight_bytes(N, K) / us / 1e3, 1),
                "pct_hbm_peak": round(100 * algo_bytes(N, K, M) / us / 1e3 / HBM_PEAK_GBS, 1),
                "int8_TOPS": round(ops / us / 1e6, 2),
                "mfma_frac": round(ops / us / 1e6 / INT8_MFMA_PEAK_TOPS, 4)}
            log(f"gemm_small M={M} {N}x{K}: {gemm[f'M{M}_{N}x{K}']}")
        # a4 at M > 1: the gate/up pair (two matrices of this shape, the
        # second half of the pool as the up projections) with relu^2
        h = torch.empty(workloads.GEMM_SMALL_M[-1], N, dtype=torch.float32, device=dev)
        half = len(P) // 2
        for M in workloads.GEMM_SMALL_M:
            xb = workloads.activations_bf16(M, K, seed=96 + M)
            xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(M, K)
            q, s = tq.tq_act_quant(xt)
            hm = h[:M]

            def fg(st, P=P, q=q, s=s, hm=hm):
                for r in range(R):
                    i = (st + r) % half
                    tq.tq_gate_up_relu2(P[i], 0.02, P[half + i], 0.03, q, s, hm)
            us = loop_us(fg, half)
            ops = 2.0 * 2 * M * N * K
            gate[f"M{M}_{N}x{K}x2"] = {
                "us_per_launch": round(us, 3),
                "weight_GBs": round(2 * weight_bytes(N, K) / us / 1e3, 1),
                "pct_hbm_peak": round(100 * 2 * weight_bytes(N, K) / us / 1e3 / HBM_PEAK_GBS, 1),
                "int8_TOPS": round(ops / us / 1e6, 2)}
            log(f"gate_up_relu2 M={M} {N}x{K}x2: {gate[f'M{M}_{N}x{K}x2']}")
        del P
    rows["gemm_small"] = gemm
    rows["gate_up_relu2_small_batch"] = gate

    # absmean ternarizer (the step before packing), 70B-class [8192, 28672]:
    # two passes over the bf16 weights (the exact mean precedes every code)
    N, K = 8192, 28672
    W = []
    for c in range(2):
        g = torch.Generator(device=dev).manual_seed(98000 + c)
        W.append((torch.randn(N, K, generator=g, device=dev) * 0.02).to(torch.bfloat16))
    pk = torch.empty(N // 4, K, dtype=torch.uint8, device=dev)
    sw = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(tq.TQ_TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    reps_t = 8

    def ft(st):
        for r in range(reps_t):
            tq.tq_ternarize(W[(st + r) % 2], pk, sw, ws)
    gs = [timer.graph(lambda s=s: ft(s)) for s in range(2)]
    us = timer.time_graphs(gs, 4) * 1e3 / reps_t
    tb = 2 * (2 * N * K) + N * K // 4
    rows["ternarize_8192x28672"] = {
        "us_per_call": round(us, 2),
        "bf16_weight_GBs": round(2 * N * K / us / 1e3, 1),
        "algo_GBs": round(tb / us / 1e3, 1),
        "pct_hbm_peak": round(100 * tb / us / 1e3 / HBM_PEAK_GBS, 1)}
    log(f"ternarize: {rows['ternarize_8192x28672']}")
    del W, gs

    # next-4: split-KV decode attention, 2B-4T heads (20 q, 5 kv, D = 128),
    # bf16 KV cache pools of >= 640 MB so repeats are not served from cache
    attn = {}
    H, Hkv, D = 20, 5, 128
    qa = torch.randn(H, D, device=dev, dtype=torch.float32)
    oa = torch.empty(H, D, device=dev, dtype=torch.float32)
    wsa = tq.attn_workspace(H, D, 131072, dev)
    for L in (2048, 8192, 32768, 131072):
        kv_bytes = 2 * L * Hkv * D * 2
        copies = max(4, -(-(640 << 20) // kv_bytes))
        g = torch.Generator(device=dev).manual_seed(99000 + L)
        KV = [(torch.randn(L, Hkv, D, generator=g, device=dev).to(torch.bfloat16),
               torch.randn(L, Hkv, D, generator=g, device=dev).to(torch.bfloat16))
              for _ in range(copies)]

        def fa(st, KV=KV):
            for r in range(R):
                kk, vv = KV[(st + r) % len(KV)]
                tq.tq_attn_decode(qa, kk, vv, out=oa, workspace=wsa)
        us = loop_us(fa, len(KV))
        ab = kv_bytes + 2 * H * D * 4
        attn[f"L{L}"] = {"us_per_call": round(us, 3),
                         "algo_GBs": round(ab / us / 1e3, 1),
                         "pct_hbm_peak": round(100 * ab / us / 1e3 / HBM_PEAK_GBS, 1)}
        log(f"attn L={L}: {attn[f'L{L}']}")
        del KV
    rows["attn_decode_2b4t_heads"] = attn

    # a6: the 30-layer decode-step chain (2B-4T layers, M = 1), one graph
    layers = []
    for l in range(workloads.CHAIN_LAYERS):
        packed, scale = {}, {}
        for name, (N, K) in workloads.LAYER_2B4T.items():
            t = workloads.TENSOR_INDEX[name]
            w = workloads.ternary_codes_torch(N, K, seed=workloads.seed_for(2, t, l), device=dev)
            packed[name] = tq.tq_pack(w)
            scale[name] = workloads.tensor_scale(t)
            del w
        layers.append(Layer(packed, scale))
    h0b = workloads.activations_bf16(1, workloads.HIDDEN, seed=97, outliers=True)
    h0 = torch.from_numpy(h0b.view(np.int16)).view(torch.bfloat16).to(dev)[0]
    layer_bytes = sum(weight_bytes(*s) for s in workloads.LAYER_2B4T.values())
    total = layer_bytes * workloads.CHAIN_LAYERS
    for fused, key, launches in ((True, "decode_chain_30x2b4t", 4),
                                 (False, "decode_chain_30x2b4t_unfused", 10)):
        chain = DecodeChain(layers, dev, fused=fused)
        g = timer.graph(lambda: chain.step(h0))
        ms = timer.time_graphs([g], 20)
        rows[key] = {
            "us_per_token": round(ms * 1e3, 2),
            "tokens_per_s": round(1e3 / ms, 1),
            "weight_GBs": round(total / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "launches_per_token": launches * workloads.CHAIN_LAYERS}
        log(f"{key}: {rows[key]}")
        del g, chain
    # the same fused chain launched eagerly (no graph): every launch goes
    # through the Python binding, so this is the host's launch rate, not the
    # GPU's -- what graph capture removes
    chain = DecodeChain(layers, dev, fused=True)
    chain.step(h0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_eager = 10
    e0.record()
    for _ in range(n_eager):
        chain.step(h0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_eager
    rows["decode_chain_30x2b4t_eager"] = {
        "us_per_token": round(ms * 1e3, 2),
        "tokens_per_s": round(1e3 / ms, 1),
        "launches_per_token": 4 * workloads.CHAIN_LAYERS,
        "note": "fused chain launched from Python without a graph (host-bound)"}
    log(f"decode_chain_30x2b4t_eager: {rows['decode_chain_30x2b4t_eager']}")
    del chain
    del layers

    # a6 at the 70B-class shapes: 8 layers (grouped q/k/v [8192,1024,1024],
    # o [8192,8192], gate/up [28672,8192], down [8192,28672]; 214 MB of
    # packed weights per layer, 1.7 GB in all), fused, one graph per step
    cfg70 = workloads.CHAIN_70B_CONFIG
    n70 = 8
    layers = []
    for l in range(n70):
        packed, scale = {}, {}
        for name, (N, K) in workloads.LAYER_70B.items():
            t = workloads.TENSOR_INDEX[name]
            w = workloads.ternary_codes_torch(N, K, seed=workloads.seed_for(cfg70, t, l),
                                              device=dev)
            packed[name] = tq.tq_pack(w)
            scale[name] = workloads.tensor_scale(t)
            del w
        layers.append(Layer(packed, scale))
    H70 = workloads.LAYER_70B["q"][1]
    h0b = workloads.activations_bf16(1, H70, seed=workloads.seed_for(cfg70, 9), outliers=True)
    h0 = torch.from_numpy(h0b.view(np.int16)).view(torch.bfloat16).to(dev)[0]
    layer_bytes = sum(weight_bytes(*s) for s in workloads.LAYER_70B.values())
    total = layer_bytes * n70
    chain = DecodeChain(layers, dev, fused=True)
    g = timer.graph(lambda: chain.step(h0))
    ms = timer.time_graphs([g], 10)
    rows["decode_chain_8x70b"] = {
        "layers": n70,
        "weight_bytes_per_layer": layer_bytes,
        "us_per_step": round(ms * 1e3, 2),
        "us_per_layer": round(ms * 1e3 / n70, 2),
        "weight_GBs": round(total / (ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
        "launches_per_layer": 4}
    log(f"decode_chain_8x70b: {rows['decode_chain_8x70b']}")
    del g, chain, layers
    return rows


if __name__ == "__main__":
    main()
