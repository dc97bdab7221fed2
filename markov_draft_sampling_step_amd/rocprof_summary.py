"""Short text summaries of rocprofv3 CSV output.

  python -m markov_draft_sampling_step_amd.rocprof_summary stats DIR
      per-kernel calls / average / min / max duration from *_kernel_stats.csv

  python -m markov_draft_sampling_step_amd.rocprof_summary counters DIR --elements N [--rank R]
      per-dispatch counter means of one --pmc run and clock-free ratios
      (VALU lane-instructions per element, VALU share of wave time, LDS
      bank-conflict stalls per LDS quad-cycle; with the MFMA counters, the
      MFMA-busy share of SIMD time and the useful share of the bf16 MFMA
      flops, 2 x elements x R)

  python -m markov_draft_sampling_step_amd.rocprof_summary traffic \\
      --fetch DIR --write DIR --copy-bytes N [--kernel markov_step_kernel]
      DRAM bytes per dispatch of the kernel from two --pmc runs (FETCH_SIZE,
      then WRITE_SIZE; the counters read KiB), each scaled by the factor that
      makes the same counter read exactly N bytes on markov_copy_kernel
      (which reads N bytes and writes N bytes).

The summaries are plain text meant to be committed; they restate the figures
the CSVs hold and print the kernel source's sha256 so that a later reader
can tell whether the measured kernel is still the current one.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "step_kernel.h")


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def stats(d: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = [f"{'kernel':48s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} "
           f"{'total %':>8s}"]
    for r in rows:
        out.append(f"{r['Name'][:48]:48s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.3f} "
                   f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                   f"{float(r['Percentage']):8.2f}")
    return "\n".join(out)


def _counter(d: str, counter: str, name_part: str) -> list[float]:
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named *{name_part}*")
    return vals


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int, kernel: str) -> str:
    cf = statistics.median(_counter(fetch_dir, "FETCH_SIZE", "markov_copy_kernel"))
    cw = statistics.median(_counter(write_dir, "WRITE_SIZE", "markov_copy_kernel"))
    kf = _counter(fetch_dir, "FETCH_SIZE", kernel)
    kw = _counter(write_dir, "WRITE_SIZE", kernel)
    f_scale = copy_bytes / cf            # bytes per counter unit, reads
    w_scale = copy_bytes / cw            # bytes per counter unit, writes
    rd = statistics.mean(kf) * f_scale
    wr = statistics.mean(kw) * w_scale
    digest = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    return "\n".join([
        f"copy calibration: markov_copy_kernel of {copy_bytes} bytes reads FETCH_SIZE={cf:.1f}, "
        f"WRITE_SIZE={cw:.1f} (KiB) -> {f_scale:.2f} and {w_scale:.2f} bytes per counter unit "
        f"(1024 would be exact KiB)",
        f"{kernel}: {len(kf)} dispatches (FETCH_SIZE run), {len(kw)} (WRITE_SIZE run); "
        f"FETCH_SIZE mean {statistics.mean(kf):.1f} min {min(kf):.1f} max {max(kf):.1f}; "
        f"WRITE_SIZE mean {statistics.mean(kw):.1f} min {min(kw):.1f} max {max(kw):.1f}",
        f"read bytes per launch  = {rd:.0f}",
        f"write bytes per launch = {wr:.0f}",
        f"traffic_bytes_per_launch = {rd + wr:.0f}",
        f"kernel_source_sha256 = {digest}",
    ])


def counters(d: str, kernel: str, elements: int, useful_flops: float = 0.0, cus: int = 256,
             xcds: int = 8) -> str:
    """Per-dispatch means of every counter of one --pmc run for the kernel,
    and three ratios that need no clock: VALU lane-instructions per (row,
    token) element (SQ_INSTS_VALU counts wave64 instructions), the share of
    wave time spent issuing VALU work (SQ_ACTIVE_INST_VALU over
    SQ_WAVE_CYCLES, both quad-cycles summed over waves), and LDS cycles
    stalled by bank conflicts per LDS-active quad-cycle."""
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"]:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id") or ""
            per.setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
            per[r["Counter_Name"]][key] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{path}: no rows for a kernel named *{kernel}*")
    mean = {c: statistics.mean(v.values()) for c, v in per.items()}
    n = len(next(iter(per.values())))
    out = [f"{kernel}: {n} dispatches; per-dispatch means (summed over the device):"]
    out += [f"  {c:28s} {mean[c]:16.1f}" for c in sorted(mean)]
    if "SQ_INSTS_VALU" in mean and elements > 0:
        out.append(f"VALU lane-instructions per element = {mean['SQ_INSTS_VALU'] * 64 / elements:.2f} "
                   f"({elements} elements per dispatch)")
    if "SQ_INSTS_MFMA" in mean and "SQ_WAVES" in mean:
        out.append(f"MFMA instructions per wave = {mean['SQ_INSTS_MFMA'] / mean['SQ_WAVES']:.1f}")
    if "SQ_ACTIVE_INST_VALU" in mean and "SQ_WAVE_CYCLES" in mean:
        out.append(f"VALU-issuing share of wave time = "
                   f"{mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_WAVE_CYCLES']:.3f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        active = mean["GRBM_GUI_ACTIVE"] / xcds           # the counter sums the XCDs
        out.append(f"MFMA-busy share of SIMD time = "
                   f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * cus * 4):.4f} "
                   f"(SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / {xcds} XCDs x {cus} CUs x 4 SIMDs)")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean and useful_flops > 0:
        done = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        out.append(f"bf16 MFMA flops per dispatch = {done:.4g} (MOPS x 512); the contraction needs "
                   f"{useful_flops:.4g} (2 rows V R): {useful_flops / done:.4f} of them are useful")
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_ACTIVE_INST_LDS" in mean:
        out.append(f"LDS bank-conflict cycles per LDS-active quad-cycle = "
                   f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_ACTIVE_INST_LDS']:.3f}")
    out.append(f"kernel_source_sha256 = {hashlib.sha256(open(KERNEL_SOURCE, 'rb').read()).hexdigest()}")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", default="markov_step_kernel")
    c.add_argument("--elements", type=int, default=0, help="(row, token) elements per dispatch")
    c.add_argument("--rank", type=int, default=0, help="R, for the useful MFMA flops 2 x elements x R")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--kernel", default="markov_step_kernel")
    args = ap.parse_args()
    if args.cmd == "stats":
        print(stats(args.dir))
    elif args.cmd == "counters":
        print(counters(args.dir, args.kernel, args.elements, 2.0 * args.elements * args.rank, args.cus,
                       args.xcds))
    else:
        print(traffic(args.fetch, args.write, args.copy_bytes, args.kernel))


if __name__ == "__main__":
    main()
