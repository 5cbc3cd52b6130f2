"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m gated_delta_rule_57_amd.profiling trace <trace_dir> <out.md> "<command>" [names]
        kernel-trace statistics (rocprofv3 --kernel-trace --stats --output-format csv);
        names, comma-separated short names, keeps only those rows
    python -m gated_delta_rule_57_amd.profiling traffic <pmc_root> <out.json> "<commands>"
        HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counter runs, each scaled by
        what the same counter reads for a device copy of 1 GiB. <pmc_root> holds the
        rocprofv3 output directories copy_FETCH_SIZE, copy_WRITE_SIZE, bench_FETCH_SIZE
        and bench_WRITE_SIZE.
    python -m gated_delta_rule_57_amd.profiling mfma <pmc_root> <trace_dir> <out.json> "<commands>"
        MFMA use per kernel from counter runs bench_<RUN> under <pmc_root> (RUN one of
        MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_MOPS_F32,
        SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES; any may be missing, and a run may
        hold several counters) and the average kernel durations of a kernel-trace run
        of the same command in <trace_dir>. The MOPS counters count MFMA work in units
        of 512 flops, so counted flops over the kernel's duration, against the chip's
        dense peak for that type, is the MFMA utilisation (mfma_util); rocprofv3's
        MfmaUtil, the fraction of SIMD cycles the MFMA unit is busy, is kept beside it
        (mfma_busy).

Kernel names are shortened to the library's kernel ids (plan, intra, inter, decode,
outnorm, bwd_local, bwd_state, bwd_chunk; seg_plan, seg_first, seg_scan and
seg_second for the segment-parallel state kernels, single_first and single_second for
the single pass, each with _gated appended for its output-epilogue variant); the
intra-chunk kernel's scalar-gate and
no-decay instantiations become intra_gdn and intra_deltanet, its 16-token-chunk
instantiation intra16, and the 16-token state kernel inter16. The general-DPLR forward's kernels are dplr_intra and dplr_inter
(the inter kernels instantiated with their DPLR flag set).
The traffic summary records a hash of the kernel sources it was taken on; bench.py
reports the traffic only while that hash matches the sources.
"""
import csv
import glob
import hashlib
import json
import os
import re
import sys

KERNELS = (("seg_plan_kernel", "seg_plan"), ("seg_scan_kernel", "seg_scan"), ("rec_seg_kernel", "seg"),
           ("seg_pass_kernel", "single"),
           ("plan_kernel", "plan"), ("dplr_intra_kernel", "dplr_intra"), ("intra_kernel", "intra"),
           ("inter_wg_kernel", "inter"),
           ("inter16_kernel", "inter16"), ("fwd_state_kernel", "inter16"), ("inter_kernel", "inter"), ("decode_kernel", "decode"),
           ("output_norm_gate_kernel", "outnorm"), ("bwd_local_kernel", "bwd_local"),
           ("bwd_state_kernel", "bwd_state"), ("bwd_chunk_kernel", "bwd_chunk"))
COPY_BYTES = 1 << 30
PEAK_FLOPS = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2.5e15, "SQ_INSTS_VALU_MFMA_MOPS_F32": 157.3e12}
# MFMA counter runs: the raw MOPS counters, and rocprofv3's derived MfmaUtil (MFMA busy
# cycles summed over SIMDs over busy GPU cycles times the SIMD count, in percent)
MFMA_RUNS = ("MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_BUSY_CU_CYCLES")
# kernels of the bf16 64-token prefill (any path) and the decode step
PREFILL_PATH = ("plan", "intra", "inter", "seg_plan", "seg_first", "seg_scan", "seg_second", "single_first",
                "single_second", "outnorm")


def kernel_source_hash(root=None):
    """Hash of the HIP sources and of the build script that sets the compiler flags,
    the same one bench.py reports."""
    root = root or os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "gated_delta_rule_57_amd")
    csrc = os.path.join(pkg, "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(csrc, n) for n in sorted(os.listdir(csrc))] + [os.path.join(pkg, "build.py")]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# the chunk and gate template arguments of intra_kernel, in mangled (..Li64ELi1EE..)
# or demangled (<.., 64, 1>) names
_GATE_ARG = re.compile(r"intra_kernel(?:I\w*?Li(\d+)ELi(\d)E|<[^>]*,\s*(\d+),\s*(\d)>)")


# the segment-parallel pass kernels' template flags, mangled (..Lb1E..) or demangled
# (<true, ..>): the second pass (the later segments), then the output-epilogue variant
# (absent from names of kernels built without it)
_PASS_FLAGS = {
    "seg": re.compile(r"rec_seg_kernel(?:ILb([01])E(?:Lb([01])E)?|<(true|false)(?:, (true|false))?>)"),
    "single": re.compile(r"seg_pass_kernel(?:ILi\d+ELb([01])E(?:Lb([01])E)?|<\d+, (true|false)(?:, (true|false))?>)"),
}


def short_name(name):
    for key, short in KERNELS:
        if key in name:
            if short in ("seg", "single"):
                m = _PASS_FLAGS[short].search(name)
                second = bool(m) and (m.group(1) == "1" or m.group(3) == "true")
                gated = bool(m) and (m.group(2) == "1" or m.group(4) == "true")
                return short + ("_second" if second else "_first") + ("_gated" if gated else "")
            if short == "intra":
                m = _GATE_ARG.search(name)
                chunk = (m.group(1) or m.group(3)) if m else None
                gate = (m.group(2) or m.group(4)) if m else None
                base = {"1": "intra_gdn", "2": "intra_deltanet"}.get(gate, "intra")
                return base + "16" if chunk == "16" else base
            if short == "inter" and (re.search(r"inter_w?g?_?kernelI\w*?Lb1E", name) or "true>" in name):
                return "dplr_inter"
            return short
    return None


def summarize_trace(trace_dir, out_md, command, names=None):
    keep = set(names.split(",")) if names else None
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(stats[0])))
    lines = ["# Kernel trace summary", "", "Command:", "", "```", command, "```", "",
             f"Kernel sources: hash {kernel_source_hash()}" + (f"; rows kept: {names}" if names else ""), "",
             "| kernel | calls | total ms | average us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        s = short_name(r["Name"])
        if s is None or (keep is not None and s not in keep):
            continue
        lines.append(f"| {s} (`{r['Name'][:60]}`) | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(run_dir, counter=None):
    """{kernel name: [value per dispatch]} of one counter, or with counter=None
    {counter: {kernel name: [...]}} of every counter in the run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if counter is not None and r["Counter_Name"] != counter:
            continue
        d = per if counter is not None else per.setdefault(r["Counter_Name"], {})
        d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_traffic(pmc_root, out_json, commands):
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = _counter(os.path.join(pmc_root, f"copy_{counter}"), counter)
        vals = [v for name, vs in copy.items() if "copyBuffer" in name for v in vs]
        if not vals:
            raise SystemExit(f"no copy kernel in the {counter} calibration run")
        kib = sum(vals) / len(vals)
        cal[counter] = {"kib_per_gib_copy": kib, "scale": (COPY_BYTES / 1024) / kib}
    kernels = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        per = _counter(os.path.join(pmc_root, f"bench_{counter}"), counter)
        for name, vs in per.items():
            s = short_name(name)
            if s is None:
                continue
            kib = sum(vs) / len(vs)
            ent = kernels.setdefault(s, {})
            ent[counter.lower() + "_kib"] = kib
            ent[counter.lower() + "_bytes_scaled"] = kib * 1024 * cal[counter]["scale"]
    for ent in kernels.values():
        ent["hbm_bytes_per_launch"] = ent.get("fetch_size_bytes_scaled", 0.0) + ent.get("write_size_bytes_scaled", 0.0)
    out = {"kernel_source_hash": kernel_source_hash(), "calibration": cal, "kernels": kernels,
           "commands": commands}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def trace_durations(trace_dir):
    """{short name: (average ns, calls)} from a kernel-trace statistics run."""
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    out = {}
    for r in csv.DictReader(open(stats[0])):
        s = short_name(r["Name"])
        if s is None:
            continue
        tot, calls = out.get(s, (0.0, 0))
        out[s] = (tot + float(r["TotalDurationNs"]), calls + int(r["Calls"]))
    return {s: (tot / calls, calls) for s, (tot, calls) in out.items()}


def summarize_mfma(pmc_root, trace_dir, out_json, commands):
    dur = trace_durations(trace_dir)
    kernels = {}
    for run_name in MFMA_RUNS:
        run = os.path.join(pmc_root, f"bench_{run_name}")
        if not os.path.isdir(run):
            continue
        for counter, by_kernel in _counter(run).items():
            for name, vs in by_kernel.items():
                s = short_name(name)
                if s is not None:
                    kernels.setdefault(s, {}).setdefault(counter, []).extend(vs)
    per = {}
    for s, cs in kernels.items():
        ent = {c: sum(v) / len(v) for c, v in cs.items()}
        if s in dur:
            ns = dur[s][0]
            ent["avg_ns"] = ns
            util = 0.0
            for c, peak in PEAK_FLOPS.items():
                if c in ent:
                    flops = ent[c] * 512
                    ent[c.replace("SQ_INSTS_VALU_MFMA_MOPS_", "mfma_flops_").lower()] = flops
                    util += flops / (ns * 1e-9) / peak
            ent["mfma_util"] = util
        if "SQ_VALU_MFMA_BUSY_CYCLES" in ent and ent.get("SQ_BUSY_CU_CYCLES"):
            ent["mfma_busy_over_cu_busy"] = ent["SQ_VALU_MFMA_BUSY_CYCLES"] / ent["SQ_BUSY_CU_CYCLES"]
        if "MfmaUtil" in ent:
            ent["mfma_busy"] = ent["MfmaUtil"] / 100.0
        per[s] = ent
    path = [s for s in PREFILL_PATH if s in per and "avg_ns" in per[s]]
    summary = None
    if path:
        ns = sum(per[s]["avg_ns"] for s in path)
        util = sum(per[s].get("mfma_util", 0.0) * per[s]["avg_ns"] for s in path) / ns
        flops = sum(per[s].get("mfma_flops_bf16", 0.0) + per[s].get("mfma_flops_f32", 0.0) for s in path)
        summary = {"prefill_kernels": path, "prefill_mfma_util": round(util, 4),
                   "prefill_mfma_flops_counted": flops, "prefill_kernel_ns": ns,
                   "per_kernel_mfma_util": {s: round(per[s].get("mfma_util", 0.0), 4) for s in path}}
        if all("mfma_busy" in per[s] for s in path):
            summary["prefill_mfma_busy"] = round(sum(per[s]["mfma_busy"] * per[s]["avg_ns"] for s in path) / ns, 4)
            summary["per_kernel_mfma_busy"] = {s: round(per[s]["mfma_busy"], 4) for s in path}
    out = {"kernel_source_hash": kernel_source_hash(), "kernels": per, "summary": summary, "commands": commands,
           "peaks_flops": PEAK_FLOPS, "mops_unit_flops": 512}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    modes = {"trace": (summarize_trace, (5, 6)), "traffic": (summarize_traffic, (5,)), "mfma": (summarize_mfma, (6,))}
    if len(sys.argv) < 2 or sys.argv[1] not in modes or len(sys.argv) not in modes[sys.argv[1]][1]:
        raise SystemExit(__doc__)
    modes[sys.argv[1]][0](*sys.argv[2:])
