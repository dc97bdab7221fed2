#!/usr/bin/env python3
"""Throughput of the Markov draft-sampling loop on one MI355X.

One bench "step" is one k-step loop (markov_sample_sequential: k kernel
launches, one per draft step) over the workload's synthetic inputs, which
are resident in HBM before timing starts. `value` is draft steps per second
(k per loop); the line also carries µs per loop, the roofline of the step
kernel and the CPU oracle's rate on a bounded sample.

Roofline: the step kernel's algorithmic HBM bytes per launch are
2VR (the w2 table) + 4 rows V (the base slice read, the cache slice
written) + 2 rows R (the rows' w1 rows); its average duration comes from
HIP events around each launch on the launching stream, over a second timed
pass of the same loops launched one step at a time.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft steps/s + µs per k-step loop, V=163840 R=256; % HBM roofline"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed k-step loops")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large",
                    choices=["tiny", "single", "small", "large", "stress"])
    ap.add_argument("--graph", action="store_true", help="replay the loop as a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="json file with measured HBM bytes per launch (from rocprofv3 counters)")
    return ap.parse_args()


def cpu_baseline(w):
    """The oracle (plain C, untuned) on a bounded sample: step 0 of the
    workload for every row, i.e. one draft step, on the host's cores."""
    import numpy as np

    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    if not os.path.exists(oracle.LIBRARY):
        oracle.build()
    t0 = time.perf_counter()
    oracle.step(np.ascontiguousarray(w.base[:, 0]), w.w1, w.w2, w.prev, w.seeds,
                w.positions[:, 0], 0, w.temperature, w.mult, w.softcap, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(1.0 / dt, 4), "unit": "draft steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"one draft step (step 0, all {w.rows} rows, V={w.V}) of the {w.name} "
                      f"workload, {threads} OpenMP threads, {dt:.2f} s wall"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Markov draft step runs on one MI355X with the "
              "full vocabulary (no sharding across GPUs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import markov_draft_sampling_step_amd as m
    from markov_draft_sampling_step_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make(args.config)
    d = workloads.to_device(w, dev)
    call = m.prepare(w, d)
    step_calls = [m.prepare(w, d, step=s) for s in range(w.k)]
    stream = torch.cuda.current_stream()

    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=side):
            call.on(side)()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # pass 1: the headline, K loops back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(args.steps):
            graph.replay()
    else:
        for _ in range(args.steps):
            call()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    loop_us = dt / args.steps * 1e6
    value = args.steps * w.k / dt

    # pass 2: the step kernel's duration, HIP events around each launch
    n2 = max(1, min(args.steps, 50))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n2 * w.k)]
    torch.cuda.synchronize()
    i = 0
    for _ in range(n2):
        for s in range(w.k):
            evs[i][0].record(stream)
            step_calls[s]()
            evs[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_us = sum(kern_ms) / len(kern_ms) * 1e3
    bytes_step = w.bytes_per_step()
    achieved = bytes_step / (kern_us * 1e-6) / 1e9

    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        traffic = json.load(open(args.traffic)).get(args.config)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "draft steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "us_per_loop": round(loop_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: V={w.V} R={w.R} rows={w.rows} k={w.k}"
                               f"{' softcap=%g' % w.softcap if w.softcap > 0 else ''}",
                   "V": w.V, "R": w.R, "rows": w.rows, "k": w.k,
                   "launches_per_loop": w.k, "mode": "graph" if graph is not None else "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(kern_us, 3),
                     "bytes_per_launch": bytes_step},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
