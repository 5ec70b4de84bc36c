"""Turn rocprofv3 output of `bench.py --step-only` into the summaries kept
under profiles/ and the traffic table bench.py reports.

    python profiling.py --stats DIR/step_kernel_stats.csv \
        --fetch DIR/pmc_counter_collection.csv --write DIR/pmc_counter_collection.csv \
        --command "<the exact rocprofv3 command>"

and the kernel table of `bench.py --components-only --component-set main`
(SwiGLU and attention at the configured shapes, one shape per kernel):

    python profiling.py --components DIR/comp_kernel_stats.csv --command "<command>"
    python profiling.py --rope-components DIR/pages_kernel_stats.csv --command "<command>"

and, from three PMC passes over the same components run, the attention
kernels' MFMA busy, VALU issue and wait fractions:

    python profiling.py --attn-counters P1.csv P2.csv P3.csv "<cmd 1>" "<cmd 2>" "<cmd 3>"

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


# attention kernels: template arguments -> (what, causal scores per launch,
# MFMA products per score of 2 D flop)
ATTN_MODES = {"0": "softcap poly FP16", "1": "softcap comparator", "2": "sigmoid poly",
              "3": "sigmoid comparator", "4": "softcap poly BF16"}
EXP_CORES = {"1": "D1", "2": "PWL2 FP16", "3": "D2", "4": "D3"}
SCORES = {"softcap": 16 * 8192 * 8193 // 2, "sigmoid": 32 * 4096 * 4097 // 2}


def attn_parts(name):
    """(kind, mode, exp2 core or None) of an attention kernel's template
    instance: k_attn_fwd<MODE, EXP, SREF>, k_attn_bwd_dq<MODE, EXP>,
    k_attn_bwd_dkdv<MODE, SPLIT, EXP>, k_attn_bwd_reduce; the stored-dS
    passes k_attn_bwd_rows and k_attn_bwd_dq_ds<NW> carry no mode."""
    import re
    m = re.search(r"k_attn_(fwd|bwd_dq_ds|bwd_dq|bwd_dkdv|bwd_reduce|bwd_rows)(?:<([^>]*)>)?", name)
    if not m:
        return None
    kind = m.group(1)
    args = [a.strip() for a in (m.group(2) or "").split(",") if a.strip()]
    mode = args[0] if args else None
    if kind in ("bwd_dq_ds", "bwd_rows"):
        return kind, None, None
    core = {"fwd": 1, "bwd_dq": 1, "bwd_dkdv": 2}.get(kind)
    exp = args[core] if core is not None and len(args) > core else None
    return kind, mode, exp if exp in EXP_CORES else None


def attn_trace_means(trace):
    """{(short name, kind, mode, exp): [ns, ...]} from a kernel trace in
    launch order.  The stored-dS passes take the mode and exp2 core of the
    dK/dV kernel of their backward call: the row pass runs just before it,
    the dQ pass just after it."""
    rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"]))
    out = collections.defaultdict(list)
    pending, last = [], None
    for r in rows:
        name = r["Kernel_Name"]
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        short_name = name.split("(")[0].replace("void ", "")
        parts = attn_parts(name)
        if parts is None:
            if "swiglu" in name:
                out[(short_name, "swiglu", None, None)].append(ns)
            continue
        kind, mode, exp = parts
        if kind == "bwd_rows":
            pending.append((short_name, ns))
            continue
        if kind == "bwd_dkdv":
            last = (mode, exp)
            for sn, v in pending:
                out[(sn, "bwd_rows", mode, exp)].append(v)
            pending = []
        if kind == "bwd_dq_ds":
            mode, exp = last if last else (None, None)
        out[(short_name, kind, mode, exp)].append(ns)
    return out


# BF16 dS bytes the dQ pass over stored blocks reads per launch: 2 KiB per
# causal 32 x 32 block
DS_BYTES = {"softcap": 16 * (256 * 257 // 2) * 2048, "sigmoid": 32 * (128 * 129 // 2) * 2048}


def components(path, command, out):
    """Kernel table of the components run from its kernel trace CSV."""
    lines = ["# SwiGLU and attention components", "",
             "Kernel trace of `bench.py --components-only --component-set main` "
             "(alternating poly / comparator rounds; softcap attention 1 x 16 x 8192 x 128 "
             "causal, sigmoid attention 1 x 32 (8 key/value heads) x 4096 x 128 causal, "
             "SwiGLU dense 8192 x 14336 and routed 131,072 x 1408 rows averaged together):",
             "", "```", command, "```", "",
             "| kernel | what | calls | mean us | MFMA TFLOP/s | % of 2.5 PF |",
             "|---|---|---|---|---|---|"]
    ds_rates = []
    means = attn_trace_means(path)
    for (short_name, kind, mode, exp), v in sorted(means.items(), key=lambda kv: (kv[0][0], str(kv[0][2]), str(kv[0][3]))):
        avg = sum(v) / len(v)
        tfl = ""
        if kind == "swiglu":
            what = "SwiGLU " + ("poly" if "Poly" in short_name else "comparator")
        else:
            what = ATTN_MODES.get(mode, "") if mode else "sum of dK/dV partials"
            if exp:
                what += f", exp2 core {EXP_CORES[exp]}"
            if kind not in ("bwd_reduce", "bwd_rows") and mode:
                fam = "softcap" if mode in "014" else "sigmoid"
                prods = {"fwd": 2, "bwd_dq": 3, "bwd_dkdv": 4, "bwd_dq_ds": 1}[kind]
                t = prods * 2 * 128 * SCORES[fam] / (avg * 1e-9) / 1e12
                tfl = f"{t:.0f} | {100 * t / 2500:.1f}"
                if kind == "bwd_dq_ds":
                    ds_rates.append(f"{what}: {DS_BYTES[fam] / avg:.0f} GB/s")
            what = f"{kind} {what}"
        lines.append(f"| `{short_name}` | {what} | {len(v)} | {avg / 1e3:.1f} | "
                     f"{tfl if tfl else '- | -'} |")
    lines += ["", "MFMA FLOP per launch counts the products each kernel performs (forward: "
              "S and PV; dq kernel: S, dP, dQ; dK/dV kernel: S, dP, dV, dK; dq_ds, the dQ pass "
              "over the stored dS blocks: dQ), 2 x 128 flop per causal score each. The "
              "stored-dS passes (bwd_rows before the dK/dV kernel, bwd_dq_ds after it) are "
              "listed under the dK/dV kernel's mode of the same backward call."]
    if ds_rates:
        lines += ["", "dS read by the dQ pass (2 KiB per causal 32 x 32 block; 1,077,936,128 bytes "
                  "softcap, 541,065,216 sigmoid): " + "; ".join(ds_rates) + "."]
    with open(os.path.join(out, "attention_components.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


ROPE_VARIANTS = {"0": "packed-FP16 D5 sine / D6 cosine", "1": "accurate sinf / cosf on the fly",
                 "2": "cached (cos, sin) table"}
ROPE_BYTES = 2 * (32 + 8) * 4096 * 128 * 2      # Q and K of 1 x 4096 x 32 (8) x 128, in and out


def rope_components(path, command, out, fetch=None, write=None, fetch_command="", write_command=""):
    """Kernel trace summary of the rotary-embedding kernels (bench.py's pages
    component set: 1 x 4096 x 32 query / 8 key heads x 128, FP16), with their
    HBM traffic when FETCH_SIZE / WRITE_SIZE passes are given (scaled by the
    factors profiles/traffic.json holds for the copy calibration)."""
    import re
    lines = ["# Rotary embedding kernels", "",
             "Kernel trace of `bench.py --components-only --component-set pages` (the fused "
             "rotary embedding of Q [1, 4096, 32, 128] and K [1, 4096, 8, 128] FP16 into the "
             "transposed layouts; 83,886,080 bytes moved per launch):", "", "```", command, "```", "",
             "| kernel | what | calls | mean us | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|"]
    for r in sorted(csv.DictReader(open(path)), key=lambda r: r["Name"]):
        m = re.search(r"k_rope<(\d)>", r["Name"])
        if not m:
            continue
        avg = float(r["AverageNs"])
        gbs = ROPE_BYTES / avg
        lines.append(f"| `pa::k_rope<{m.group(1)}>` | {ROPE_VARIANTS[m.group(1)]} | {r['Calls']} | "
                     f"{avg / 1e3:.2f} | {gbs:.0f} | {100 * gbs / 8000:.1f} |")
    if fetch and write:
        cal = json.load(open(os.path.join(out, "traffic.json")))["calibration"]
        per = {}
        for pth, key in ((fetch, "f"), (write, "w")):
            acc = collections.defaultdict(list)
            for r in csv.DictReader(open(pth)):
                m = re.search(r"k_rope<(\d)>", r["Kernel_Name"])
                if m:
                    acc[m.group(1)].append(float(r["Counter_Value"]))
            for k, v in acc.items():
                per.setdefault(k, {})[key] = sum(v) / len(v)
        lines += ["", "HBM traffic per launch (PMC FETCH_SIZE and WRITE_SIZE in separate runs, KiB "
                  f"per dispatch scaled by the copy calibration: x{cal['fetch_factor']:.4f} and "
                  f"x{cal['write_factor']:.4f}):", "", "```", fetch_command, write_command, "```", "",
                  "| kernel | read B | written B | algorithmic B | ratio |", "|---|---|---|---|---|"]
        for k in sorted(per):
            rd = per[k].get("f", 0.0) * 1024 * cal["fetch_factor"]
            wr = per[k].get("w", 0.0) * 1024 * cal["write_factor"]
            lines.append(f"| `pa::k_rope<{k}>` | {rd:,.0f} | {wr:,.0f} | {ROPE_BYTES:,} | "
                         f"{(rd + wr) / ROPE_BYTES:.4f} |")
    with open(os.path.join(out, "rope_components.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def per_dispatch_counters(path):
    """{kernel short name: {counter: mean over dispatches of the per-dispatch sum}}"""
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in rows:
        k = short(r["Kernel_Name"])
        if not k:
            continue
        agg[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = k
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, cs in agg.items():
        for c, v in cs.items():
            out[names[d]][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in out.items()}


def counters(specs, out):
    """specs: (elements, VALU-pass csv, L2-pass csv, VALU command, L2 command)"""
    lines = ["# Elementwise FP16 kernels: VALU busy and L2 hit rate", "",
             "PMC passes (one counter group per run, no tracing) over the timed steps of "
             "`bench.py --step-only` at the two endpoints of the isolated sweep. VALUBusy is "
             "rocprofv3's derived metric (100 x SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE); "
             "VALU instructions are per wave, i.e. per 512 elements (one 16-byte chunk per "
             "lane); the L2 hit rate is TCC_HIT / (TCC_HIT + TCC_MISS).", ""]
    for n, vpath, lpath, vcmd, lcmd in specs:
        v, l2 = per_dispatch_counters(vpath), per_dispatch_counters(lpath)
        lines += [f"## {n:,} elements", "", "```", vcmd, lcmd, "```", "",
                  "| kernel | bench name | VALUBusy % | VALU instructions per wave | L2 hit % |",
                  "|---|---|---|---|---|"]
        for k, (names, _) in KERNELS.items():
            if k not in v or k not in l2:
                continue
            waves = n / 512
            hit = l2[k].get("TCC_HIT_sum", 0.0)
            miss = l2[k].get("TCC_MISS_sum", 0.0)
            lines.append(f"| `{k}` | {', '.join(names)} | {v[k].get('VALUBusy', float('nan')):.1f} | "
                         f"{v[k].get('SQ_INSTS_VALU', float('nan')) / waves:.1f} | "
                         f"{100 * hit / max(hit + miss, 1):.1f} |")
        lines.append("")
    with open(os.path.join(out, "elementwise_counters.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


CLOCK_HZ = 2.4e9      # MI355X peak engine clock (MFMA-busy fractions assume it)
SIMDS = 256 * 4


def attn_label(kind, mode, exp):
    what = ATTN_MODES.get(mode, "")
    if exp:
        what += f", exp2 core {EXP_CORES[exp]}"
    return f"{kind} {what}"


def attn_pass(path):
    """{label: (summed counters over the label's dispatches, summed ns)} of one
    PMC pass; the dQ pass over stored dS takes the mode of the dK/dV kernel
    dispatched before it (the row pass is left out: no MFMA)"""
    rows = list(csv.DictReader(open(path)))
    kinds = {}
    for r in rows:
        parts = attn_parts(r["Kernel_Name"])
        if parts and parts[0] not in ("bwd_reduce", "bwd_rows"):
            kinds[int(r["Dispatch_Id"])] = parts
    labels, last = {}, None
    for d in sorted(kinds):
        kind, mode, exp = kinds[d]
        if kind == "bwd_dkdv":
            last = (mode, exp)
        if kind == "bwd_dq_ds":
            if last is None:
                continue
            mode, exp = last
        labels[d] = attn_label(kind, mode, exp)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    span = {}
    for r in rows:
        lab = labels.get(int(r["Dispatch_Id"]))
        if not lab:
            continue
        per[lab][r["Counter_Name"]] += float(r["Counter_Value"])
        span[(lab, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    ns = collections.defaultdict(float)
    for (lab, _), d in span.items():
        ns[lab] += d
    return {lab: (cs, ns[lab]) for lab, cs in per.items()}


def attn_counters(paths, commands, out):
    """paths / commands: the three PMC passes (wave states; MFMA and
    instruction counts; L2 and LDS conflicts)."""
    p1, p2, p3 = (attn_pass(p) for p in paths)
    lines = ["# Attention kernels: MFMA busy, VALU issue and waits", "",
             "PMC passes (one counter group per run, no tracing) over "
             "`bench.py --components-only --component-set main --protocol quick` (softcap "
             "attention 1 x 16 x 8192 x 128 causal, sigmoid attention 1 x 32 (8) x 4096 x 128 "
             "causal, forward and backward):", "", "```"] + list(commands) + ["```", "",
             "MFMA busy and MFMA/VALU co-execution: SQ_VALU_MFMA_BUSY_CYCLES and "
             "SQ_VALU_MFMA_COEXEC_CYCLES over the dispatches' duration x 1,024 SIMDs x 2.4 GHz "
             "(the peak clock, so a lower clock under the profiler would read lower). Per wave "
             "(fractions of SQ_WAVE_CYCLES): VALU issue SQ_ACTIVE_INST_VALU, LDS issue "
             "SQ_ACTIVE_INST_LDS, waiting on s_waitcnt SQ_WAIT_ANY, instruction-issue stalls "
             "SQ_WAIT_INST_ANY. VALU / MFMA is SQ_INSTS_VALU / SQ_INSTS_MFMA. L2 hit rate "
             "TCC_HIT / (TCC_HIT + TCC_MISS); LDS bank conflicts as cycles per LDS-active cycle.", "",
             "| kernel | MFMA busy % | co-exec % | VALU issue % | LDS issue % | s_waitcnt % | "
             "issue stall % | VALU / MFMA | L2 hit % | LDS conflict % |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for lab in sorted(set(p1) & set(p2) & set(p3)):
        c1, _ = p1[lab]
        c2, ns2 = p2[lab]
        c3, _ = p3[lab]
        simd_cycles = ns2 * 1e-9 * CLOCK_HZ * SIMDS
        wc = max(c1.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        hit, miss = c3.get("TCC_HIT_sum", 0.0), c3.get("TCC_MISS_sum", 0.0)
        lines.append(
            f"| {lab} | {100 * c2.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / simd_cycles:.1f} | "
            f"{100 * c2.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0) / simd_cycles:.1f} | "
            f"{100 * c1.get('SQ_ACTIVE_INST_VALU', 0) / wc:.1f} | "
            f"{100 * c1.get('SQ_ACTIVE_INST_LDS', 0) / wc:.1f} | "
            f"{100 * c1.get('SQ_WAIT_ANY', 0) / wc:.1f} | "
            f"{100 * c1.get('SQ_WAIT_INST_ANY', 0) / wc:.1f} | "
            f"{c2.get('SQ_INSTS_VALU', 0) / max(c2.get('SQ_INSTS_MFMA', 0), 1):.1f} | "
            f"{100 * hit / max(hit + miss, 1):.1f} | "
            f"{100 * c3.get('SQ_LDS_BANK_CONFLICT', 0) / max(c3.get('SQ_LDS_IDX_ACTIVE', 0), 1):.2f} |")
    with open(os.path.join(out, "attention_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--components", default="")
    ap.add_argument("--rope-components", default="")
    ap.add_argument("--attn-counters", nargs=6, default=None,
                    metavar=("CSV1", "CSV2", "CSV3", "COMMAND1", "COMMAND2", "COMMAND3"),
                    help="attention counter summary from three PMC passes")
    ap.add_argument("--counters", nargs=5, action="append", default=[],
                    metavar=("ELEMENTS", "VALU_CSV", "L2_CSV", "VALU_COMMAND", "L2_COMMAND"),
                    help="VALU busy / L2 hit rate summary for one step size (repeatable)")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--command", default="")
    ap.add_argument("--fetch-command", default="")
    ap.add_argument("--write-command", default="")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.attn_counters:
        attn_counters(a.attn_counters[:3], a.attn_counters[3:], a.out)
        return
    if a.counters:
        counters([(int(c[0]),) + tuple(c[1:]) for c in a.counters], a.out)
        return
    if a.components:
        components(a.components, a.command, a.out)
        return
    if a.rope_components:
        rope_components(a.rope_components, a.command, a.out, a.fetch, a.write, a.fetch_command,
                        a.write_command)
        return
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
