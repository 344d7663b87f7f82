"""Benchmark of the ternary GEMV hot path at M = 1 on one MI355X.

A step is one pass of the hot path over the workload the metric names:
for each of the shapes [N, K] = [2560, 6912] (2B-4T down projection),
[28672, 8192] and [8192, 28672] (70B-class layer, both orientations):
per-token int8 quantization of a bf16 activation (tq_act_quant), then the
ternary GEMV with its fp32 rescale (tq_gemv).  Weights are seeded synthetic
ternary codes (P(0) = 0.35), packed on the GPU; activations are bf16 N(0,1).

Measurement:
  * Weights come from a pool of distinct buffers (>= 1 GiB) cycled step by
    step, so the 256 MB Infinity Cache cannot serve repeats.
  * Each pool set's step is captured in a HIP graph; the timed region replays
    K graphs.  A spin kernel queued just before the start event keeps the host
    ahead of the GPU, so HIP events measure GPU execution only.
  * The dominant kernel (the GEMV instantiation that runs both 70B-class
    shapes) is timed per launch with event pairs on its stream; its
    algorithmic bytes (packed weights + int8 activations + scale + fp32
    outputs) over that time give roofline.achieved against 8 TB/s.
  * cpu_baseline: the CPU oracle (plain C, one thread) on the same step for
    one pool set, repeated for about 10 s.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("ternary GEMV weight GB/s + % of MI355X HBM peak at M=1 "
          "(2560x6912, 8192x28672)")
SHAPES = {"down_2b4t": (2560, 6912), "70b_up": (28672, 8192),
          "70b_down": (8192, 28672)}
DOMINANT = ("70b_up", "70b_down")
HBM_PEAK_GBS = 8000.0
POOL_BYTES_MIN = 1 << 30
COUNTER_FILE = os.path.join(ROOT, "profiles", "tq_gemv_70b_counters.txt")
KERNEL_SOURCES = ("bit_gemv_tq_amd/csrc/tq_gemv.hip",
                  "bit_gemv_tq_amd/csrc/tq_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(N, K):
    return N * K // 4


def algo_bytes(N, K):
    # packed weights + int8 activations + fp32 x_scale + fp32 outputs
    return N * K // 4 + K + 4 + 4 * N


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per dominant-kernel launch from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(COUNTER_FILE):
        return None
    fields = {}
    for line in open(COUNTER_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(budget_s=10.0):
    """The CPU oracle on one step of the same workload (one pool set)."""
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
    reps, t0 = 0, time.perf_counter()
    while True:
        for name, (N, K) in SHAPES.items():
            q, s = oracle.act_quant(xbits[name], "bf16")
            oracle.gemv(packed[name], s_w, q, s, N)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    step_bytes = sum(weight_bytes(*s) for s in SHAPES.values())
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": (f"{reps} full steps (all three shapes, act_quant + GEMV) "
                       f"in {el:.1f} s, one thread, {platform.processor() or platform.machine()}, "
                       f"{os.cpu_count()} host cores visible")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU-oracle baseline leg")
    ap.add_argument("--kernel-reps", type=int, default=100,
                    help="per-shape event-timed launches for the kernel table")
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
    s_w = np.float32(0.02)

    # ---------------------------------------------------------------- pool
    set_bytes = sum(weight_bytes(*s) for s in SHAPES.values())
    n_sets = max(2, -(-POOL_BYTES_MIN // set_bytes))
    log(f"building weight pool: {n_sets} sets x {set_bytes / 1e6:.1f} MB")
    pool = []
    for i in range(n_sets):
        d = {}
        for t, (name, (N, K)) in enumerate(SHAPES.items()):
            w = workloads.ternary_codes_torch(N, K, seed=workloads.seed_for(4, t, i) + 7919,
                                              device=dev)
            d[name] = tq.tq_pack(w)
            del w
        pool.append(d)
    torch.cuda.synchronize()
    x, xq, xs, y = {}, {}, {}, {}
    for t, (name, (N, K)) in enumerate(SHAPES.items()):
        xb = workloads.activations_bf16(1, K, seed=workloads.seed_for(4, 20 + t))
        x[name] = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)[0]
        xq[name] = torch.empty(K, dtype=torch.int8, device=dev)
        xs[name] = torch.empty(1, dtype=torch.float32, device=dev)
        y[name] = torch.empty(N, dtype=torch.float32, device=dev)

    def step(i, stream=None):
        P = pool[i % n_sets]
        for name in SHAPES:
            tq.tq_act_quant(x[name], xq[name], xs[name], stream=stream)
            tq.tq_gemv(P[name], s_w, xq[name], xs[name], y[name], stream=stream)

    # ---------------------------------------------------------------- graphs
    log("capturing step graphs")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(n_sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        graphs[i % n_sets].replay()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    spin = 50_000_000  # ~20 ms of spinning: the host queues ahead meanwhile
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    torch.cuda._sleep(spin)
    ev0.record()
    for i in range(args.steps):
        graphs[i % n_sets].replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    step_wbytes = set_bytes
    value = step_wbytes / (ms_step * 1e-3) / 1e9

    # ------------------------------------------------- per-kernel timing
    # Event pairs around single launches on the current stream, queued
    # behind a spin so that the host is ahead of the GPU.
    per_shape = {}
    stream = torch.cuda.current_stream()
    evs = {name: [(torch.cuda.Event(enable_timing=True),
                   torch.cuda.Event(enable_timing=True))
                  for _ in range(args.kernel_reps)] for name in SHAPES}
    for name in SHAPES:
        tq.tq_act_quant(x[name], xq[name], xs[name])
    torch.cuda.synchronize()
    torch.cuda._sleep(spin)
    for r in range(args.kernel_reps):        # same order and pool walk as a step
        for name in SHAPES:
            a, b = evs[name][r]
            a.record(stream)
            tq.tq_gemv(pool[r % n_sets][name], s_w, xq[name], xs[name], y[name])
            b.record(stream)
    torch.cuda.synchronize()
    for name, (N, K) in SHAPES.items():
        times = [a.elapsed_time(b) * 1e3 for a, b in evs[name]]   # us
        mean_us = float(np.mean(times))
        per_shape[name] = {
            "N": N, "K": K, "us_mean": round(mean_us, 3),
            "us_median": round(float(np.median(times)), 3),
            "weight_GBs": round(weight_bytes(N, K) / mean_us / 1e3, 1),
            "pct_hbm_peak": round(100 * weight_bytes(N, K) / mean_us / 1e3 / HBM_PEAK_GBS, 1),
        }
        log(f"{name}: {per_shape[name]}")

    dom_bytes = sum(algo_bytes(*SHAPES[n]) for n in DOMINANT)
    dom_us = sum(per_shape[n]["us_mean"] for n in DOMINANT)
    achieved = dom_bytes / dom_us / 1e3  # GB/s
    traffic = read_traffic()

    cpu = None if args.no_cpu else cpu_baseline()

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
            "workload": "ternary GEMV at M=1 over [N,K] = [2560,6912], [28672,8192], "
                        "[8192,28672]; each shape act_quant(bf16) + gemv per step",
            "weight_bytes_per_step": step_wbytes,
            "pool_sets": n_sets,
            "pool_bytes": n_sets * set_bytes,
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_m1_kernel (70B-class shapes)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "per_shape": per_shape,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
