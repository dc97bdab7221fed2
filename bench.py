#!/usr/bin/env python3
"""Throughput of the Markov draft-sampling loop on one MI355X.

One bench "step" is one k-step loop (markov_sample_sequential: one step
kernel launch per draft step; the last one also writes the last tokens) over the workload's
synthetic inputs, which are resident in HBM before timing starts. `value` is
draft steps per second (k per loop) of the headline mode, plain launches
(eager); the same loop captured once as a HIP graph and replayed is reported
beside it (on this part a replay measures no faster than the eager loop). The line also carries the step kernel's roofline and the CPU
oracle's rate on a bounded sample.

Roofline: the step kernel's algorithmic HBM bytes per launch are
2VR (the w2 table) + 4 rows V (the base slice read, the cache slice
written) + 2 rows R (the rows' w1 rows); its average duration comes from
HIP events recorded around each step-kernel launch on the launching stream,
in a timed pass of eager loops. Measured DRAM traffic (rocprofv3 FETCH_SIZE
and WRITE_SIZE, scaled by the same counters on a plain copy) is read from
the committed profile summary and reported only while the kernel source is
the one it was measured on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft steps/s + µs per k-step loop, V=163840 R=256; % HBM roofline"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "markov_draft_sampling_step_amd", "csrc", "step_kernel.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "markov_step_kernel_{cfg}{path}_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed k-step loops")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large",
                    choices=["tiny", "single", "small", "large", "stress"])
    ap.add_argument("--rows", type=int, default=0,
                    help="override the config's row count (same distributions; for the small-row "
                         "contraction sweep)")
    ap.add_argument("--path", default="sample",
                    choices=["sample", "greedy", "greedy-chain", "fp8", "fp8-greedy", "shard",
                             "verify-greedy", "verify-prob"],
                    help="sample: markov_sample_sequential (the headline); greedy: "
                         "markov_greedy_sequential writing the cache; greedy-chain: the same "
                         "without the cache write; fp8 / fp8-greedy: the same two with the E4M3 "
                         "w2 (quantized once, untimed); shard: one GPU's share of a vocabulary-"
                         "parallel loop (markov_shard_step on slab 0 of --shards, then "
                         "markov_pick over the shards' packets, per step)")
    ap.add_argument("--verify-rows", type=int, default=64,
                    help="batch rows of --path verify-* (P = 5 proposals, V = 163840)")
    ap.add_argument("--shards", type=int, default=8,
                    help="vocabulary slabs of --path shard (one GPU's share is timed)")
    ap.add_argument("--graph", action="store_true",
                    help="headline from replays of the loop captured as a HIP graph")
    ap.add_argument("--eager", action="store_true",
                    help="plain launches only (no graph capture at all)")
    ap.add_argument("--cold", action="store_true",
                    help="also time loops with a 1 GiB write between them (MALL evicted)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-time budget of the CPU oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device copies (markov_copy_kernel) of MIB MiB, the "
                         "reference for the DRAM byte counters")
    return ap.parse_args()


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(cfg: str, kpath: str = "sample"):
    """DRAM bytes per step-kernel launch from the committed counter summary,
    or None when there is none or the kernel source changed since."""
    path = TRAFFIC_SUMMARY.format(cfg=cfg, path="" if kpath == "sample" else "_" + kpath.replace("-", "_"))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch\s*=\s*(\d+)", text)
    h = re.search(r"kernel_source_sha256\s*=\s*([0-9a-f]{64})", text)
    if not m or not h or h.group(1) != source_digest():
        return None
    return int(m.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """The oracle (plain C, untuned) on a bounded sample of the workload.

    Leg 1: whole k-step loops over every row, repeated until the wall-time
    budget is spent, on the host threads a GPU machine gives one GPU (16; its
    OpenMP loop runs over rows). Leg 2: one thread, one draft step over the
    first rows (a slice of about a second), extrapolated to draft steps/s of
    the whole workload (rows are independent and cost the same)."""
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    used = min(threads, w.rows)
    if not os.path.exists(oracle.LIBRARY):
        oracle.build()
    loops = 0
    t0 = time.perf_counter()
    while True:
        oracle.sample_sequential(w.base, w.w1, w.w2, w.prev, w.seeds, w.positions,
                                 w.temperature, w.mult, w.softcap, threads=threads)
        loops += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or loops >= 1000:
            break
    # single thread: one step over n1 rows, n1 grown until it takes ~1 s
    n1, t1 = 1, 0.0
    while True:
        rows = np.arange(min(n1, w.rows))
        t = time.perf_counter()
        oracle.step(np.ascontiguousarray(w.base[rows, 0]), w.w1, w.w2, w.prev[rows],
                    w.seeds[rows], w.positions[rows, 0], 0, w.temperature[rows], w.mult,
                    w.softcap, threads=1)
        t1 = time.perf_counter() - t
        if t1 >= 1.0 or n1 >= w.rows:
            break
        n1 = min(w.rows, n1 * 2)
    single = (len(rows) / w.rows) / t1          # whole-workload draft steps/s, one thread
    return {"value": round(loops * w.k / dt, 4), "unit": "draft steps/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{loops} whole {w.k}-step loop(s) of the {w.name} workload (all {w.rows} "
                      f"rows, V={w.V}), {used} OpenMP thread(s) over rows, {dt:.2f} s wall",
            "single_thread": {"value": round(single, 5), "unit": "draft steps/s",
                              "sample": f"one draft step of {len(rows)} of {w.rows} rows on one "
                                        f"thread in {t1:.2f} s, extrapolated to all rows"}}


def percentile(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


def time_loops(torch, launch, stream, n):
    """n loops back to back: (wall µs per loop, per-loop event µs)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n * 1e6
    return wall, [a.elapsed_time(b) * 1e3 for a, b in evs]


def bench_verify(args, torch, m, workloads, dev, stream):
    """One verifier launch per bench step over the synthetic drafted block
    (64 rows, 5 proposals, V = 163840); value = verified rows per second.
    Algorithmic bytes: the greedy verifier reads target positions 0..L of
    each row (bf16), the probabilistic one the p and q rows of the first
    rejection (or p_L) once (fp32)."""
    v = workloads.make_verify(B=args.verify_rows)
    B, P, V = v.B, v.P, v.V
    acc = torch.empty((B, P + 1), dtype=torch.int64, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    ws = m.new_verify_workspace(B, P, device=dev)
    L = torch.from_numpy(v.lengths).to(dev)
    if args.path == "verify-greedy":
        lg = torch.from_numpy(v.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        dr = torch.from_numpy(v.draft_greedy).to(dev)
        call = lambda: m.greedy_accept(lg, dr, L, acc, n, ws)   # noqa: E731
    else:
        t = torch.from_numpy(v.target).to(dev)
        q = torch.from_numpy(v.draftp).to(dev)
        dr = torch.from_numpy(v.draft_sampled).to(dev)
        u = torch.from_numpy(v.uniforms).to(dev)
        call = lambda: m.prob_accept(t, q, dr, L, u, acc, n, ws)   # noqa: E731
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    wall, ev = time_loops(torch, call, stream, args.steps)
    kern_us = sum(ev) / len(ev)
    nl = n.cpu().numpy()
    Lc = np.clip(v.lengths, 0, P)
    if args.path == "verify-greedy":
        bytes_launch = int(((Lc + 1) * 2 * V).sum())
    else:
        rejected = nl <= Lc                      # the token after the accepted drafts was resampled
        bytes_launch = int(np.where(rejected, 8 * V, 4 * V).sum())
    achieved = bytes_launch / (kern_us * 1e-6) / 1e9
    out = {
        "metric": "verified rows/s (" + args.path + ")", "value": round(B / (wall * 1e-6), 1),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e-3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if args.path == "verify-greedy" else "f32",
        "data": "synthetic",
        "config": {"workload": f"verify: B={B} P={P} V={V}", "path": args.path, "mode": "eager"},
        "us_per_launch_p10_p50_p90": [round(percentile(ev, q), 2) for q in (0.1, 0.5, 0.9)],
        "accept_lengths": np.bincount(nl, minlength=P + 2).tolist(),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_us": round(kern_us, 3), "bytes_per_launch": bytes_launch,
                     "kernel": "greedy_accept_kernel" if args.path == "verify-greedy"
                     else "prob_accept_kernel"},
    }
    print(json.dumps(out), flush=True)


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
    stream = torch.cuda.current_stream()

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            m.debug_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    if args.path.startswith("verify"):
        return bench_verify(args, torch, m, workloads, dev, stream)

    w = workloads.make(args.config, rows=args.rows or None)
    d = workloads.to_device(w, dev)
    bytes_step = w.bytes_per_step()
    if args.path == "sample":
        call = m.prepare(w, d)
        step_calls = [m.prepare(w, d, step=s) for s in range(w.k)]
    elif args.path.startswith("fp8"):
        q = torch.empty((w.V, w.R), dtype=torch.uint8, device=dev)
        sc = torch.empty(w.V, dtype=torch.int16, device=dev)
        m.quantize_w2_fp8(d["w2"], q, sc)
        torch.cuda.synchronize()
        d["w2q"], d["w2s"] = q, sc
        greedy = args.path == "fp8-greedy"
        call = m.prepare_fp8(w, d, greedy=greedy)
        step_calls = [m.prepare_fp8(w, d, greedy=greedy, step=s) for s in range(w.k)]
        bytes_step -= w.V * w.R - 2 * w.V       # 1-byte codes and a 2-byte scale per row
    elif args.path == "shard":
        G = args.shards
        Vs = w.V // G
        base0 = d["base"][:, :, :Vs].contiguous()
        w20 = d["w2"][:Vs].contiguous()
        cache0 = torch.empty((w.rows, w.k, Vs), dtype=torch.bfloat16, device=dev)
        ws0 = m.new_workspace(w.rows, Vs, w.R, w.k, device=dev, mult=w.mult, softcap=w.softcap)
        packets = torch.zeros((G, w.rows), dtype=torch.int64, device=dev)
        flat = d["tokens"].view(-1)

        def shard_call(s):
            def f():
                feed, stride = (d["prev"], 1) if s == 0 else (flat[s - 1:], w.k)
                m.shard_step(base0, d["w1"], w20, feed, d["seeds"], d["positions"],
                             d["temperature"], cache0, packets[0], ws0, step=s, vocab_offset=0,
                             feed_stride=stride, mult=w.mult, softcap=w.softcap)
            return f

        def pick_call(s):
            return lambda: m.pick(packets, flat[s:], stride=w.k)

        step_calls = [shard_call(s) for s in range(w.k)]
        picks = [pick_call(s) for s in range(w.k)]

        def call():
            for s in range(w.k):
                step_calls[s]()
                picks[s]()
        call.on = None
        bytes_step = 2 * Vs * w.R + 4 * w.rows * Vs + 2 * w.rows * w.R
    else:
        chain = args.path == "greedy-chain"
        call = m.prepare_greedy(w, d, cache=not chain)
        step_calls = [m.prepare_greedy(w, d, cache=not chain, step=s) for s in range(w.k)]
        if chain:
            bytes_step -= 2 * w.rows * w.V       # no cache slice written
    launches = w.k                           # one step kernel per draft step

    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()

    graph = None
    if not args.eager and args.path != "shard":
        side = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            call.on(side)()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()

    # the timed loops: graph replays (unless --eager) and eager launches, K each
    g_wall, g_ev = time_loops(torch, graph.replay, stream, args.steps) if graph else (None, None)
    e_wall, e_ev = time_loops(torch, call, stream, args.steps)
    head_wall, head_ev = (g_wall, g_ev) if (graph and args.graph) else (e_wall, e_ev)
    value = w.k / (head_wall * 1e-6)

    # the step kernel alone: events around each step-kernel launch of eager
    # loops, every step index (the last one also turns the winners into
    # tokens); the average over all k launches is the roofline's duration
    n2 = max(1, min(args.steps, 50))
    evs = [[] for _ in range(w.k)]
    torch.cuda.synchronize()
    for _ in range(n2):
        for s in range(w.k):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step_calls[s]()
            b.record(stream)
            evs[s].append((a, b))
    torch.cuda.synchronize()
    per_step = [sum(a.elapsed_time(b) for a, b in e) / len(e) * 1e3 for e in evs]
    kern_us = sum(per_step) / len(per_step)
    achieved = bytes_step / (kern_us * 1e-6) / 1e9

    cold = None
    if args.cold:
        junk = torch.empty(1 << 29, dtype=torch.float16, device=dev)
        ts = []
        for _ in range(min(args.steps, 20)):
            junk.fill_(1.0)
            torch.cuda.synchronize()
            _, ev = time_loops(torch, graph.replay if (graph and args.graph) else call, stream, 1)
            ts += ev
        cold = round(percentile(ts, 0.5), 2)
        del junk

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "draft steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_wall * 1e-3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: V={w.V} R={w.R} rows={w.rows} k={w.k}"
                               f"{' softcap=%g' % w.softcap if w.softcap > 0 else ''}",
                   "V": w.V, "R": w.R, "rows": w.rows, "k": w.k,
                   "launches_per_loop": launches * (2 if args.path == "shard" else 1),
                   "path": args.path,
                   **({"shards": args.shards, "slab_vocab": w.V // args.shards}
                      if args.path == "shard" else {}),
                   "mode": "graph" if (graph and args.graph) else "eager"},
        "us_per_loop": round(head_wall, 2),
        "us_per_loop_p10_p50_p90": [round(percentile(head_ev, q), 2) for q in (0.1, 0.5, 0.9)],
        "us_per_loop_graph": round(g_wall, 2) if graph else None,
        "us_per_loop_eager": round(e_wall, 2),
        "us_per_loop_cold": cold,
        "draft_tokens_per_s": round(w.rows * value, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.config, args.path), "kernel_us": round(kern_us, 3),
                     "kernel_us_per_step_index": [round(x, 3) for x in per_step],
                     "bytes_per_launch": bytes_step, "kernel": "markov_step_kernel"},
    }
    if not args.no_cpu_baseline and args.path == "sample":
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
