"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m gated_delta_rule_57_amd.profiling trace <trace_dir> <out.md> "<command>" [names]
        kernel-trace statistics (rocprofv3 --kernel-trace --stats --output-format csv);
        names, comma-separated short names, keeps only those rows
    python -m gated_delta_rule_57_amd.profiling traffic <pmc_root> <out.json> "<commands>"
        HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counter runs, each scaled by
        what the same counter reads for a device copy of 1 GiB. <pmc_root> holds the
        rocprofv3 output directories copy_FETCH_SIZE, copy_WRITE_SIZE, bench_FETCH_SIZE
        and bench_WRITE_SIZE.

Kernel names are shortened to the library's kernel ids (plan, intra, inter, decode,
outnorm, bwd_local, bwd_state, bwd_chunk); the intra-chunk kernel's scalar-gate and
no-decay instantiations become intra_gdn and intra_deltanet, its 16-token-chunk
instantiation (the backward's forward pass) intra16, and the 16-token state
kernel inter16. The general-DPLR forward's kernels are dplr_intra and dplr_inter
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

KERNELS = (("plan_kernel", "plan"), ("dplr_intra_kernel", "dplr_intra"), ("intra_kernel", "intra"),
           ("inter_wg_kernel", "inter"),
           ("inter16_kernel", "inter16"), ("fwd_state_kernel", "inter16"), ("inter_kernel", "inter"), ("decode_kernel", "decode"),
           ("output_norm_gate_kernel", "outnorm"), ("bwd_local_kernel", "bwd_local"),
           ("bwd_state_kernel", "bwd_state"), ("bwd_chunk_kernel", "bwd_chunk"))
COPY_BYTES = 1 << 30


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


def short_name(name):
    for key, short in KERNELS:
        if key in name:
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


def _counter(run_dir, counter):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
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


if __name__ == "__main__":
    if len(sys.argv) not in (5, 6) or sys.argv[1] not in ("trace", "traffic") or \
            (sys.argv[1] == "traffic" and len(sys.argv) != 5):
        raise SystemExit(__doc__)
    {"trace": summarize_trace, "traffic": summarize_traffic}[sys.argv[1]](*sys.argv[2:])
