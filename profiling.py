"""Turn rocprofv3 output of `bench.py --step-only` into the summaries kept
under profiles/ and the traffic table bench.py reports.

    python profiling.py --stats DIR/step_kernel_stats.csv \
        --fetch DIR/pmc_counter_collection.csv --write DIR/pmc_counter_collection.csv \
        --command "<the exact rocprofv3 command>"

Traffic calibration: the FETCH_SIZE / WRITE_SIZE derived counters are scaled
by what they read for the device-to-device hipMemcpy of x (536,870,912 bytes
read and written) issued at the end of the profiled run: factor = true bytes /
counter bytes, per counter.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))
N = 268_435_456
COPY_BYTES = 2 * N          # the FP16 array x: bytes read and bytes written by its copy
# kernel template instance -> bench names and algorithmic bytes per element
KERNELS = {
    "PolyFwdF16<1, 3>": (["sigmoid_fwd"], 4),
    "PolyFwdF16<2, 4>": (["tanh_fwd"], 4),
    "PolyFwdF16<3, 3>": (["silu_fwd"], 4),
    "PolyFwdF16<4, 5>": (["gelu_fwd"], 4),
    "PolyBwdF16<4>": (["sigmoid_bwd", "tanh_bwd"], 6),
}


def short(name):
    for k in KERNELS:
        if k in name:
            return k
    return None


def per_dispatch(path):
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    copy = []
    for r in rows:
        v = float(r["Counter_Value"]) * 1024.0        # KiB -> bytes
        if "copyBuffer" in r["Kernel_Name"]:
            copy.append((int(r["Dispatch_Id"]), v))
        k = short(r["Kernel_Name"])
        if k:
            agg[k].append(v)
    last_copy = max(copy)[1]
    return {k: sum(v) / len(v) for k, v in agg.items()}, last_copy


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--fetch-command", default="")
    ap.add_argument("--write-command", default="")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    import sys
    sys.path.insert(0, ROOT)
    from elementwise_symmetry_range_amd._build import source_digest

    stats = {}
    for r in csv.DictReader(open(a.stats)):
        k = short(r["Name"])
        if k:
            stats[k] = (int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]))
    fetch, fcopy = per_dispatch(a.fetch)
    write, wcopy = per_dispatch(a.write)
    ff, fw = COPY_BYTES / fcopy, COPY_BYTES / wcopy

    lines = ["# Elementwise FP16 kernels, 268,435,456 elements (HBM resident)", "",
             "Kernel trace (rocprofv3 --kernel-trace --stats) of the timed steps of "
             "`bench.py --step-only`:", "", "```", a.command, "```", "",
             "| kernel | bench name | calls | mean ns | min ns | max ns | algorithmic GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|"]
    for k, (names, bpe) in KERNELS.items():
        if k not in stats:
            continue
        c, avg, mn, mx = stats[k]
        gbs = bpe * N / avg
        lines.append(f"| `{k}` | {', '.join(names)} | {c} | {avg:.0f} | {mn:.0f} | {mx:.0f} | "
                     f"{gbs:.1f} | {100 * gbs / 8000:.1f} |")
    lines += ["", "## HBM traffic (PMC FETCH_SIZE / WRITE_SIZE, separate runs)", ""]
    if a.fetch_command:
        lines += ["```", a.fetch_command, a.write_command, "```", ""]
    lines += [f"Calibration on the device-to-device hipMemcpy of x ({COPY_BYTES:,} bytes each "
              f"way): FETCH_SIZE reads {fcopy / 1024:,.0f} KiB -> factor {ff:.4f}; WRITE_SIZE reads "
              f"{wcopy / 1024:,.0f} KiB -> factor {fw:.4f}.", "",
              "| kernel | FETCH KiB | WRITE KiB | scaled read B | scaled write B | algorithmic B | ratio |",
              "|---|---|---|---|---|---|---|"]
    traffic = {}
    for k, (names, bpe) in KERNELS.items():
        if k not in fetch:
            continue
        rd, wr = fetch[k] * ff, write[k] * fw
        alg = bpe * N
        lines.append(f"| `{k}` | {fetch[k] / 1024:,.0f} | {write[k] / 1024:,.0f} | {rd:,.0f} | "
                     f"{wr:,.0f} | {alg:,} | {(rd + wr) / alg:.4f} |")
        for nm in names:
            traffic[nm] = int(round(rd + wr))
    digest = source_digest()
    lines += ["", f"Kernel sources digest: `{digest}`."]
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, "elementwise_f16_268M.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(a.out, "traffic.json"), "w") as f:
        json.dump({"source_digest": digest, "unit": "bytes per launch", "kernels": traffic,
                   "calibration": {"fetch_factor": ff, "write_factor": fw}}, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
