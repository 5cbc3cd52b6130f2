"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill over a 131072-token sequence with 32 heads of
dimension 128 (bf16 q/k/v, fp32 decays and state, chunk 64, the library's automatic
kernel choice), followed by ``--decode-per-step`` decode steps over 256 sequences x
32 heads of persisted fp32 128 x 128 states (bf16 q/k/v). Inputs are synthetic,
seeded (NumPy on the host, see gated_delta_rule_57_amd/inputs.py) and resident in
HBM before timing starts.

Prints one JSON line. ``value`` is prefill tokens/s (a token = one position across
all 32 heads) from the median of the timed steps' prefill durations, measured with
events on the stream the library's kernels run on. Beside it:
  roofline      the whole prefill path against the HBM roofline: the method's
                algorithmic bytes (q, k, v, log_alpha, beta in, o out: 1,540 B per
                token and head) over the measured time, against 8 TB/s
  mfma          algorithmic bf16 TFLOP/s and fraction of the 2.5 PFLOP/s dense peak;
                the rocprof MFMA utilisation from the committed counter summary
  kernels       each kernel of the path: average time, its design bytes (what it
                moves by construction) and the HBM traffic measured by the counters
  decode, configs, paths, fused, gates, backward, dplr_comparison, cpu_baseline(s),
  environment

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import glob
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA

D = 128
CHUNK = 64
# algorithmic flops per (token, head) of the chunked prefill at C = 64, d = 128 (triangles
# counted exactly): state products 6 d^2, A (C-1) d, P (C+1) d, P U~ (C+1) d, T [bK | bV] (C-1) 2d
FLOP_PER_TOK_HEAD = 6 * D * D + (CHUNK - 1) * D + (CHUNK + 1) * D + (CHUNK + 1) * D + (CHUNK - 1) * 2 * D
# bytes every prefill must move per (token, head): q, k, v bf16, log_alpha fp32, beta fp32, o bf16
PATH_BYTES_PER_TOK_HEAD = 3 * 2 * D + 4 * D + 4 + 2 * D
IN_BYTES_PER_TOK_HEAD = 3 * 2 * D + 4 * D + 4
# per-(chunk, head) record written by the intra-chunk kernel: its size in the workspace, and
# the bytes it writes (the two all-zero P slots above the diagonal, 2 x 1 KiB, are not written)
RECORD_BYTES_BF16_C64 = 74240
RECORD_MOVED_BYTES_BF16_C64 = RECORD_BYTES_BF16_C64 - 2048
# what the segment-parallel state kernels read per chunk: the output pass the whole
# record (fragment region, e^{g_C}, U), a map pass -W, (K e^{g_C-G})^T, e^{g_C} and the
# U tiles of its B columns
SEG_OUT_READ = RECORD_BYTES_BF16_C64
SEG_MAP_READ = 16384 + 16384 + 512 + 16384
# segment length rule of the library (SEG_TARGET_GROUPS, SEG_MIN_CHUNKS, SEG_FIRST_PCT_* in
# kda_internal.h): the first segment of a sequence is a share of the later ones
SEG_TARGET_GROUPS, SEG_MIN_CHUNKS = 256, 1
SEG_FIRST_PCT = {("record", False): 55, ("single", False): 80, ("record", True): 42, ("single", True): 70}
# one decode (sequence, head): fp32 state read + written, q, k, v bf16, log_alpha fp32, beta, o bf16
DECODE_BYTES_PER_HEAD = 2 * 4 * D * D + 3 * 2 * D + 4 * D + 4 + 2 * D

# backward (16-token chunks, bf16): per (chunk, head) the forward state pass's record
# (-W 4096 B, (K e^{g_C-G})^T 8192 B, U 4096 B, e^{g_C} 512 B: 16896 B), the backward
# record (13312 B), the chunk-entry state and the chunk-end state gradient
# (2 x 32768 B), U~, dU~ (2 x 4096 B) and T, M (2 x 16 x 16 fp32); per (token, head)
# algorithmic bytes of each kernel
BWD_CHUNK = 16
BWD_FWD_RECORD = 16896
BWD_TM_BYTES = 2 * 16 * 16 * 4
BWD_BYTES_PER_TOK_HEAD = {
    "bwd_local": 3 * 2 * D + 4 * D + 4 + (13312 + BWD_FWD_RECORD + BWD_TM_BYTES) // BWD_CHUNK,  # inputs in, records out
    "inter": BWD_FWD_RECORD // BWD_CHUNK + (32768 + 4096) // BWD_CHUNK,     # record in, states and U~ out
    "bwd_state": 13312 // BWD_CHUNK + 2 * D + (32768 + 4096) // BWD_CHUNK,  # record, grad_o in, dS_C, dU~ out
    "bwd_chunk": 4 * 2 * D + 4 * D + 4 + (2 * (32768 + 4096) + BWD_TM_BYTES) // BWD_CHUNK + 3 * 2 * D + 4 * D + 4,
}
# bytes any backward must move per (token, head): q, k, v, grad_o, log_alpha, beta in; the five gradients out
BWD_PATH_BYTES_PER_TOK_HEAD = 4 * 2 * D + 4 * D + 4 + 3 * 2 * D + 4 * D + 4

# general DPLR forward (64-token chunks, bf16): per (chunk, head) record of 123392 B
DPLR_RECORD_BYTES_BF16 = 123392
DPLR_RECORD_MOVED_BYTES_BF16 = DPLR_RECORD_BYTES_BF16 - 2048
DPLR_IN_BYTES_PER_TOK_HEAD = 5 * 2 * D + 4 * D   # q, k, v, a, b bf16, log_alpha fp32

PREFILL_T, PREFILL_H = 131072, 32
DEC_N, DEC_H = 256, 32
PREFILL_KERNELS = ("plan", "intra", "inter", "seg_first", "seg_scan", "seg_second", "outnorm")


def stats(xs):
    xs = sorted(xs)
    return {"median": round(statistics.median(xs), 5), "min": round(xs[0], 5), "max": round(xs[-1], 5),
            "runs": len(xs)}


def kernel_source_hash():
    from gated_delta_rule_57_amd.profiling import kernel_source_hash as source_hash
    return source_hash(ROOT)


def committed_profile(name, src_hash):
    """A committed counter summary under profiles/, if it was taken on the current
    kernel sources; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    return data if data.get("kernel_source_hash") == src_hash else None


def seg_plan(T, H, N=1, kernels="record", gated=False):
    """The library's segment plan for N sequences of T tokens and H heads: (chunks per
    segment after the first, chunks in the first, segments per sequence); gated: with
    the output epilogue, whose output chunks cost more."""
    pct = SEG_FIRST_PCT[(kernels, gated)]
    nc = (T + CHUNK - 1) // CHUNK
    mc = N * nc
    den = SEG_TARGET_GROUPS * 100 + N * H * pct
    lseg = max(SEG_MIN_CHUNKS, (mc * H * 100 + den - 1) // den)
    lseg = min(lseg, mc) if mc > 0 else 1
    l0 = max(1, (lseg * pct + 99) // 100)
    ns = 1 if nc <= l0 else 1 + (nc - l0 + lseg - 1) // lseg
    return lseg, l0, ns


def seg_design_bytes(T, H, kernels="record"):
    """Bytes the segment-parallel passes read and write by construction for one T-token
    sequence of H heads: (first pass, second pass). Record-fed: a record and o per
    output chunk, the map parts of the record per middle chunk. Single pass: the inputs
    and o per output chunk, the inputs but q per middle chunk."""
    lseg, l0, ns = seg_plan(T, H, kernels=kernels)
    nc = (T + CHUNK - 1) // CHUNK
    lens = [min(l0, nc)] + [min(lseg, nc - l0 - (j - 1) * lseg) for j in range(1, ns)]
    o_per_chunk = CHUNK * 2 * D
    if kernels == "single":
        out_chunk = CHUNK * (IN_BYTES_PER_TOK_HEAD + 2 * D)
        map_chunk = CHUNK * (IN_BYTES_PER_TOK_HEAD - 2 * D)
    else:
        out_chunk = SEG_OUT_READ + o_per_chunk
        map_chunk = SEG_MAP_READ
    first = H * (lens[0] * out_chunk + sum(lens[1:ns - 1]) * map_chunk)
    second = H * sum(lens[1:]) * out_chunk
    return first, second


def environment(torch):
    env = {"python": platform.python_version(), "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None)}
    try:
        p = torch.cuda.get_device_properties(0)
        arch = getattr(p, "gcnArchName", None)
        env.update(gpu=p.name or (arch.split(":")[0] if arch else None), gcn_arch=arch,
                   compute_units=p.multi_processor_count, hbm_gib=round(p.total_memory / 2**30, 1))
        clk = getattr(p, "clock_rate", None)
        if clk:
            env["gpu_clock_mhz"] = round(clk / 1000)
    except Exception:  # noqa: BLE001 (best-effort environment record)
        pass
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            env["rocm"] = open(path).read().strip()
            break
        except OSError:
            pass
    try:
        env["amdgpu_driver"] = open("/sys/module/amdgpu/version").read().strip()
    except OSError:
        pass
    # current shader and memory clock levels (the '*' entry of the DPM tables), read
    # from sysfs so no other program is started from this GPU process
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        for key, name in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
            try:
                cur = [ln.strip() for ln in open(os.path.join(os.path.dirname(path), name)) if "*" in ln]
            except OSError:
                continue
            if cur:
                env.setdefault("dpm_clocks", {})[key] = cur[0]
        if "dpm_clocks" in env:
            break
    env.update(host_cpu=cpu_model(), host_cores=host_cores(), omp_num_threads=os.environ.get("OMP_NUM_THREADS"))
    return env


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count()


class StreamTimer:
    """Event pairs on the current stream (the one the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def __call__(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def time_fn(torch, fn, runs, warmup=2):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    tm = StreamTimer(torch)
    for _ in range(runs):
        tm("x", fn)
    torch.cuda.synchronize()
    return tm.ms("x")


def cpu_baselines(inputs, pre, dec):
    """The fp64 sequential oracle (the C recurrence of oracle/, OpenMP over sequences,
    heads and 16-column blocks) on this host: the headline workload, the 4K and varlen
    workloads, one thread on the 4K workload, and decode steps of the decode workload."""
    import numpy as np
    import oracle
    threads = oracle.seq.default_threads()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    out = {}

    def prefill(label, inp, tokens=None, nt=threads):
        S = inp.q.shape[1] if tokens is None else min(tokens, inp.q.shape[1])
        x = [f(t[:, :S]) for t in (inp.q, inp.k, inp.v, inp.log_alpha, inp.beta)]
        s0 = None if inp.initial_state is None else inp.initial_state.double().cpu().numpy()
        cu = None if inp.cu_seqlens is None else inp.cu_seqlens.cpu().numpy().astype(np.int64)
        t0 = time.perf_counter()
        o, _ = oracle.forward(*x, s0, cu_seqlens=cu, num_threads=nt)
        dt = time.perf_counter() - t0
        assert np.isfinite(o).all()
        out[label] = {"tokens_per_s": round(S * inp.q.shape[0] / dt, 1), "seconds": round(dt, 3), "threads": nt,
                      "tokens": S * inp.q.shape[0], "heads": inp.q.shape[2]}
        print(f"[bench] oracle {label}: {dt:.2f} s", file=sys.stderr, flush=True)

    prefill("kda_prefill_T131072_H32_bf16", pre)
    w1 = inputs.make_workload(1, device="cpu")
    prefill("kda_prefill_T4096_H16_bf16", w1)
    prefill("kda_prefill_T4096_H16_bf16_one_thread", w1, nt=1)
    prefill("kda_varlen_4seq_T32768_H32_bf16", inputs.make_workload(2, device="cpu"))
    steps = 32
    state = dec.initial_state.double().cpu().numpy()
    t0 = time.perf_counter()
    for i in range(steps):
        oracle.decode_step(f(dec.q[i]), f(dec.k[i]), f(dec.v[i]), f(dec.log_alpha[i]), f(dec.beta[i]), state,
                           num_threads=threads)
    dt = time.perf_counter() - t0
    out["kda_decode_N256_H32_bf16"] = {"tokens_per_s": round(DEC_N * steps / dt, 1), "seconds": round(dt, 3),
                                       "threads": threads, "steps": steps}
    print(f"[bench] oracle decode: {dt:.2f} s", file=sys.stderr, flush=True)
    return out, threads


def config_timing(inputs, kda, torch, dev, runs=20):
    """The other prefill workloads on the GPU: the fp32 64-token latency case and the
    4K and varlen throughput cases (median / min / max over ``runs``)."""
    res = {}
    w0 = inputs.make_workload(0, device=dev)
    o = torch.empty_like(w0.v)
    fin = torch.empty(1, 1, D, D, dtype=torch.float32, device=dev)
    ws0 = torch.empty(kda.workspace_size(1, 64, 1, 0, 16, kda.KDA_FP32), dtype=torch.uint8, device=dev)
    call0 = lambda: kda.chunk_fwd(w0.q, w0.k, w0.v, w0.log_alpha, w0.beta, chunk=16, o=o,  # noqa: E731
                                  final_state=fin, workspace=ws0)
    ms = time_fn(torch, call0, runs=50)
    kda.timing_enable(True)
    time_fn(torch, call0, runs=50)
    kt = kda.timing_read()
    kda.timing_enable(False)
    # end to end: events around each call (library timing off), so the host's launch work
    # between them counts; kernels: the library's own per-kernel event times, in a second
    # set of runs
    res["kda_fwd_T64_H1_fp32_c16"] = {
        "latency_us": {k: (round(v * 1e3, 2) if k != "runs" else v) for k, v in stats(ms).items()},
        "kernel_us": {n: round(tot / cnt * 1e3, 2) for n, (tot, cnt) in kt.items() if cnt}}
    for idx in (1, 2):
        w = inputs.make_workload(idx, device=dev)
        B, T, H = w.q.shape[:3]
        n = w.num_seqs if w.cu_seqlens is not None else 0
        ws = torch.empty(kda.workspace_size(B, T, H, n, 64, kda.KDA_BF16), dtype=torch.uint8, device=dev)
        o = torch.empty_like(w.v)
        fin = torch.empty(w.num_seqs, H, D, D, dtype=torch.float32, device=dev)
        ms = time_fn(torch, lambda: kda.chunk_fwd(w.q, w.k, w.v, w.log_alpha, w.beta, initial_state=w.initial_state,
                                                  cu_seqlens=w.cu_seqlens, chunk=64, o=o, final_state=fin,
                                                  workspace=ws), runs=runs)
        st = stats(ms)
        med = st["median"] * 1e-3
        res[inputs.WORKLOADS[idx]["name"]] = {
            "ms": st, "tokens_per_s": round(B * T / med, 1),
            "path_hbm_frac": round(PATH_BYTES_PER_TOK_HEAD * B * T * H / med / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] {inputs.WORKLOADS[idx]['name']}: {st['median']:.3f} ms", file=sys.stderr, flush=True)
        del w, ws, o, fin
    torch.cuda.empty_cache()
    return res


def path_timing(kda, torch, pre, runs=20):
    """The headline prefill on each kernel set (kda_prefill_path)."""
    B, T, H = pre.q.shape[:3]
    out = {}
    for path in ("record", "segmented", "single"):
        ws = torch.empty(kda.workspace_size(B, T, H, 0, 64, kda.KDA_BF16, path=path), dtype=torch.uint8,
                         device=pre.q.device)
        o = torch.empty_like(pre.v)
        fin = torch.empty(B, H, D, D, dtype=torch.float32, device=pre.q.device)

        def run():
            kda.chunk_fwd(pre.q, pre.k, pre.v, pre.log_alpha, pre.beta, chunk=CHUNK, o=o, final_state=fin,
                          workspace=ws, path=path)
        run()
        torch.cuda.synchronize()
        kda.timing_enable(True)
        ms = time_fn(torch, run, runs=runs, warmup=0)
        t = kda.timing_read()
        kda.timing_enable(False)
        km = {n: round(tot / cnt, 4) for n, (tot, cnt) in t.items() if cnt}
        med = statistics.median(ms)
        out[path] = {"ms": round(med, 4), "tokens_per_s": round(T / (med * 1e-3), 1), "kernel_ms": km,
                     "workspace_bytes": ws.numel()}
        print(f"[bench] path {path}: {med:.3f} ms", file=sys.stderr, flush=True)
        del ws, o, fin
    torch.cuda.empty_cache()
    return out


def fused_timing(inputs, kda, torch, dev, pre, dec, state, o_dec, runs=20):
    """The fused layer core on the same shapes: the prefill on raw q, k and gate /
    beta pre-activations with the output RMSNorm and gate, and the fused decode
    step."""
    B, T, H = pre.q.shape[:3]
    raw = inputs.make_raw_prefill(3, B=B, T=T, H=H, dtype="bf16", device=dev)
    fu = kda.fusion(out_gate=raw.out_gate, norm_weight=raw.norm_weight)
    z_dec = torch.randn(o_dec.shape, device=dev).to(o_dec.dtype)
    fu_dec = kda.fusion(out_gate=z_dec, norm_weight=raw.norm_weight)
    o = torch.empty_like(pre.v)
    fin = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(B, T, H, 0, 64, kda.KDA_BF16), dtype=torch.uint8, device=dev)
    prefill = lambda: kda.chunk_fwd(raw.q, raw.k, raw.v, raw.gate, raw.beta, chunk=CHUNK, o=o,  # noqa: E731
                                    final_state=fin, workspace=ws, fusion=fu)
    pms = time_fn(torch, prefill, runs=runs)
    dms = time_fn(torch, lambda: kda.decode_step(dec.q[0], dec.k[0], dec.v[0], dec.log_alpha[0], dec.beta[0],
                                                 state, o=o_dec, fusion=fu_dec), runs=16)
    med = statistics.median(pms)
    dec_bytes = DEC_N * DEC_H * (DECODE_BYTES_PER_HEAD + 2 * D)
    print(f"[bench] fused prefill {med:.3f} ms", file=sys.stderr, flush=True)
    del raw, o, fin, ws
    torch.cuda.empty_cache()
    return {"workload": "kda_prefill_T131072_H32_bf16 raw inputs (q, k unnormalised; gate and beta "
                        "pre-activations; output RMSNorm and sigmoid gate) + kda_decode_N256_H32_bf16",
            "prefill_ms": stats(pms), "tokens_per_s": round(T / (med * 1e-3), 1),
            "decode_ms_per_step": stats(dms),
            "decode_GBps": round(dec_bytes / (statistics.median(dms) * 1e-3) / 1e9, 1)}


def gate_timing(kda, torch, pre, dec, state, o_dec, runs=20):
    """The scalar-gate (one decay per token and head) and no-decay paths on the
    headline prefill shape and the decode batch."""
    B, T, H = pre.q.shape[:3]
    la_head = pre.log_alpha[..., 0].contiguous()
    la_dec = dec.log_alpha[..., 0].contiguous()
    o = torch.empty_like(pre.v)
    fin = torch.empty(B, H, D, D, dtype=torch.float32, device=pre.q.device)
    ws = torch.empty(kda.workspace_size(B, T, H, 0, 64, kda.KDA_BF16), dtype=torch.uint8, device=pre.q.device)
    out = {}
    for name, la, lad in (("gated_deltanet", la_head, la_dec), ("deltanet", None, None)):
        pms = time_fn(torch, lambda: kda.chunk_fwd(pre.q, pre.k, pre.v, la, pre.beta, chunk=CHUNK, o=o,
                                                   final_state=fin, workspace=ws), runs=runs)
        dms = time_fn(torch, lambda: kda.decode_step(dec.q[0], dec.k[0], dec.v[0], None if lad is None else lad[0],
                                                     dec.beta[0], state, o=o_dec), runs=16)
        med = statistics.median(pms)
        out[name] = {"prefill_ms": stats(pms), "tokens_per_s": round(T / (med * 1e-3), 1),
                     "decode_ms_per_step": stats(dms)}
        print(f"[bench] {name} prefill {med:.3f} ms", file=sys.stderr, flush=True)
    del o, fin, ws
    torch.cuda.empty_cache()
    return out


def backward_timing(inputs, kda, torch, pre, runs=20):
    """The backward (kda_chunk_bwd) on the headline prefill shape: gradients of q, k,
    v, log_alpha, beta and the initial state for a random output cotangent and a
    final-state cotangent, timed by the library's events."""
    B, T, H = pre.q.shape[:3]
    grad_o, gfin = inputs.make_cotangents(3, pre)
    ws = torch.empty(kda.bwd_workspace_size(B, T, H, dtype=kda.KDA_BF16), dtype=torch.uint8, device=pre.q.device)

    def run():
        return kda.chunk_bwd(pre.q, pre.k, pre.v, pre.log_alpha, pre.beta, grad_o, initial_state=pre.initial_state,
                             grad_final_state=gfin, workspace=ws)

    g = run()
    torch.cuda.synchronize()
    del g
    kda.timing_enable(True)
    calls = time_fn(torch, run, runs=runs, warmup=0)  # events around each whole call
    t = kda.timing_read()
    kda.timing_enable(False)
    g = run()
    torch.cuda.synchronize()
    ms = {n: tot / max(cnt, 1) for n, (tot, cnt) in t.items() if cnt}
    names = ("plan", "bwd_local", "inter", "bwd_state", "bwd_chunk")
    total = sum(ms.get(n, 0.0) for n in names)
    tok_heads = T * H
    gbps = {n: round(BWD_BYTES_PER_TOK_HEAD[n] * tok_heads / (ms[n] * 1e-3) / 1e9, 1)
            for n in names if n in BWD_BYTES_PER_TOK_HEAD and n in ms}
    finite = all(bool(torch.isfinite(x).all()) for x in g.values() if x is not None)
    del g, ws, grad_o
    torch.cuda.empty_cache()
    print(f"[bench] backward {total:.3f} ms", file=sys.stderr, flush=True)
    return {"workload": "kda_backward_T131072_H32_bf16 (gradients of q, k, v, log_alpha, beta and the initial "
                        "state; 16-token chunks)",
            "ms": round(total, 4), "tokens_per_s": round(T / (total * 1e-3), 1),
            "call_ms": stats(calls),  # whole calls, output allocation included
            "kernel_ms": {n: round(ms.get(n, 0.0), 4) for n in names},
            "kernel_GBps_design": gbps,
            "path_hbm_frac": round(BWD_PATH_BYTES_PER_TOK_HEAD * tok_heads / (total * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "finite": finite}


def dplr_comparison(inputs, kda, torch, dev, pre, lengths=(4096, 16384, 65536, 131072), runs=20):
    """KDA's chunked forward against the general DPLR chunked forward
    (kda_dplr_chunk_fwd) on the same shapes: H = 32, d = 128, bf16, 64-token chunks,
    over input lengths. KDA runs the same kernel structure as the DPLR forward (the
    record path: intra-chunk records, slab state kernels) and, beside it, its automatic
    path. Prefixes of one 131072-token input set per method (KDA: the headline workload;
    DPLR: the stable tied recipe with the same mixed decays)."""
    B, Tmax, H = pre.q.shape[:3]
    x = inputs.make_dplr(3, B=1, T=Tmax, H=H, dtype="bf16", la_mode="mixed", device=dev)
    ws_d = torch.empty(kda.dplr_workspace_size(1, Tmax, H, 0, kda.KDA_BF16), dtype=torch.uint8, device=dev)
    ws_k = torch.empty(kda.workspace_size(1, Tmax, H, 0, 64, kda.KDA_BF16, path="record"), dtype=torch.uint8,
                       device=dev)
    ws_a = torch.empty(kda.workspace_size(1, Tmax, H, 0, 64, kda.KDA_BF16), dtype=torch.uint8, device=dev)
    o = torch.empty_like(pre.v)
    fin = torch.empty(1, H, D, D, dtype=torch.float32, device=dev)
    rows = []
    for T in lengths:
        if T > Tmax:
            continue
        sl = lambda t: t[:, :T]  # noqa: E731
        kr = statistics.median(time_fn(torch, lambda: kda.chunk_fwd(
            sl(pre.q), sl(pre.k), sl(pre.v), sl(pre.log_alpha), sl(pre.beta), chunk=CHUNK, o=o[:, :T],
            final_state=fin, workspace=ws_k, path="record"), runs=runs))
        ka = statistics.median(time_fn(torch, lambda: kda.chunk_fwd(
            sl(pre.q), sl(pre.k), sl(pre.v), sl(pre.log_alpha), sl(pre.beta), chunk=CHUNK, o=o[:, :T],
            final_state=fin, workspace=ws_a), runs=runs))
        dm = statistics.median(time_fn(torch, lambda: kda.dplr_chunk_fwd(
            sl(x.q), sl(x.k), sl(x.v), sl(x.a), sl(x.b), sl(x.log_alpha), o=o[:, :T], final_state=fin,
            workspace=ws_d), runs=runs))
        rows.append({"T": T, "kda_record_ms": round(kr, 4), "kda_auto_ms": round(ka, 4), "dplr_ms": round(dm, 4),
                     "dplr_over_kda_same_kernels": round(dm / kr, 3), "dplr_over_kda_auto": round(dm / ka, 3),
                     "kda_tokens_per_s": round(T / (ka * 1e-3), 1), "dplr_tokens_per_s": round(T / (dm * 1e-3), 1)})
        print(f"[bench] T={T}: kda {kr:.3f} / {ka:.3f} ms, dplr {dm:.3f} ms", file=sys.stderr, flush=True)
    del x, ws_d, ws_k, ws_a, o, fin
    torch.cuda.empty_cache()
    return {"workload": "kda_vs_dplr_H32_bf16_c64 (prefill at several lengths; the general DPLR transition "
                        "Diag(alpha) + a b^T with free a, b against KDA's key-tied one)",
            "lengths": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-per-step", type=int, default=8)
    ap.add_argument("--decode-inputs", type=int, default=256, help="distinct decode tokens, cycled")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=("auto", "record", "segmented", "single"),
                    help="prefill kernel set of the headline steps (kda_prefill_path)")
    ap.add_argument("--extras", default="configs,paths,fused,gates,backward,dplr",
                    help="comma-separated sections timed after the headline steps")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline steps (no configs, paths, fused, gates, backward, DPLR)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-dplr", action="store_true", help="skip the KDA versus general-DPLR comparison")
    ap.add_argument("--dplr-lengths", default="4096,16384,65536,131072",
                    help="comma-separated sequence lengths of the DPLR comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device copy of 1 GiB (for counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the KDA path "
              "here has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_57_amd import inputs, kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        nbytes = 1 << 30
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)
        return

    t_gen = time.perf_counter()
    pre = inputs.make_workload(3, device=dev)
    dec = inputs.make_decode(N=DEC_N, H=DEC_H, n_steps=args.decode_inputs, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    B, T, H = pre.q.shape[:3]
    ws = torch.empty(kda.workspace_size(B, T, H, 0, CHUNK, kda.KDA_BF16, path=args.path), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(pre.v)
    fin = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    state = dec.initial_state.clone()
    o_dec = torch.empty(DEC_N, DEC_H, D, dtype=torch.bfloat16, device=dev)
    n_dec_in = dec.q.shape[0]
    dec_i = [0]
    tm = StreamTimer(torch)

    def prefill():
        kda.chunk_fwd(pre.q, pre.k, pre.v, pre.log_alpha, pre.beta, chunk=CHUNK, o=o, final_state=fin, workspace=ws,
                      path=args.path)

    def decode():
        i = dec_i[0] % n_dec_in
        kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], state, o=o_dec)
        dec_i[0] += 1

    def step(timed):
        if timed:
            tm("prefill", prefill)
            for _ in range(args.decode_per_step):
                tm("decode", decode)
        else:
            prefill()
            for _ in range(args.decode_per_step):
                decode()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    kda.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timing = kda.timing_read()
    kda.timing_enable(False)
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    K = args.steps
    pst, dst = stats(tm.ms("prefill")), stats(tm.ms("decode"))
    prefill_ms, dec_ms = pst["median"], dst["median"]
    tokens_per_s = T / (prefill_ms * 1e-3)
    tok_heads = T * H
    kms = {n: tot / cnt for n, (tot, cnt) in timing.items() if cnt}
    src_hash = kernel_source_hash()
    # counters of the default kernel set, and of the single pass in a file of its own
    traffic = committed_profile("pmc_traffic.json" if args.path in ("auto", "segmented")
                                else f"pmc_traffic_{args.path}.json", src_hash)
    mfma_prof = committed_profile("pmc_mfma.json", src_hash)

    # the whole prefill path against the HBM roofline, on the method's bytes
    path_bytes = PATH_BYTES_PER_TOK_HEAD * tok_heads
    flops = FLOP_PER_TOK_HEAD * tok_heads
    achieved = path_bytes / (prefill_ms * 1e-3) / 1e9
    t_bound_ms = max(flops / (BF16_MFMA_PEAK_TFLOPS * 1e12), path_bytes / (HBM_PEAK_GBS * 1e9)) * 1e3
    path_kernels = [n for n in PREFILL_KERNELS if n in kms]
    # the single pass runs under the segment kernels' timing slots; its counters are
    # kept under names of its own
    kernel_set = "single" if args.path == "single" else "record"
    prof_name = {"seg_first": "single_first", "seg_second": "single_second"} if kernel_set == "single" else {}
    path_traffic = None
    if traffic:
        per = traffic.get("kernels", {})
        names = {prof_name.get(n, n) for n in path_kernels} | ({"seg_plan"} if "seg_first" in path_kernels else set())
        if all(n in per for n in names):
            path_traffic = round(sum(per[n]["hbm_bytes_per_launch"] for n in names), 0)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": path_traffic,
            "kernel": "prefill path (" + ", ".join(path_kernels) + ")",
            "algorithmic_bytes": path_bytes, "t_bound_ms": round(t_bound_ms, 4),
            "frac_t_bound_over_t": round(t_bound_ms / prefill_ms, 4)}

    # each kernel of the path: design bytes (what it moves by construction) and counter traffic
    n_chunks = (T + CHUNK - 1) // CHUNK
    rec_moved = n_chunks * H * RECORD_MOVED_BYTES_BF16_C64
    seg_a, seg_b = seg_design_bytes(T, H, kernels=kernel_set)
    lseg, l0, ns = seg_plan(T, H, kernels=kernel_set)
    design = {"intra": tok_heads * IN_BYTES_PER_TOK_HEAD + rec_moved,
              "inter": rec_moved + tok_heads * 2 * D,
              "seg_first": seg_a, "seg_second": seg_b,
              # each of a head's 8 column work-groups reads a middle segment's whole M and
              # its slice of B and writes its slice of the next entry state
              "seg_scan": H * (max(0, ns - 2) * 10 + 1) * 4 * D * D,
              "decode": DEC_N * DEC_H * DECODE_BYTES_PER_HEAD}
    share = {"intra": tok_heads * IN_BYTES_PER_TOK_HEAD}  # the method's bytes each kernel is responsible for
    share["seg_second" if "seg_second" in kms else "inter"] = tok_heads * 2 * D
    kernels = {}
    for name in path_kernels + ["decode"]:
        avg = kms[name]
        ent = {"avg_ms": round(avg, 4), "launches": timing[name][1]}
        if name in design:
            ent["design_bytes_per_launch"] = design[name]
            ent["design_GBps"] = round(design[name] / (avg * 1e-3) / 1e9, 1)
            ent["design_frac_of_hbm_peak"] = round(design[name] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if name in share:
            ent["algorithmic_bytes_per_launch"] = share[name]
        pname = prof_name.get(name, name)
        if traffic and pname in traffic.get("kernels", {}):
            tb = traffic["kernels"][pname]["hbm_bytes_per_launch"]
            ent["traffic_bytes"] = round(tb, 0)
            if name in design:
                ent["traffic_over_design"] = round(tb / design[name], 3)
            if name in share:
                ent["traffic_over_algorithmic"] = round(tb / share[name], 3)
        kernels[name] = ent

    dec_gbs = DEC_N * DEC_H * DECODE_BYTES_PER_HEAD / (dec_ms * 1e-3) / 1e9
    mfma = {"algorithmic_tflops": round(flops / (prefill_ms * 1e-3) / 1e12, 2),
            "algorithmic_frac_of_bf16_peak": round(flops / (prefill_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "mfma_util_rocprof": None, "rocprof": None}
    if mfma_prof and mfma_prof.get("summary"):
        mfma["rocprof"] = mfma_prof["summary"]
        mfma["mfma_util_rocprof"] = mfma_prof["summary"].get("prefill_mfma_util")
        mfma["mfma_busy_rocprof"] = mfma_prof["summary"].get("prefill_mfma_busy")

    result = {
        "metric": "KDA prefill tokens/s (H=32,d=128) + %MFMA peak; decode GB/s %HBM peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_prefill_T131072_H32_bf16", "T": T, "H": H, "d": D, "chunk": CHUNK,
                   "decode_workload": "kda_decode_N256_H32_bf16", "decode_per_step": args.decode_per_step,
                   "prefill_path": args.path, "parallelism": "single GPU"},
        "prefill": {"ms": pst, "tokens_per_s": round(tokens_per_s, 1),
                    "path_hbm_frac": roof["frac"],
                    "kernel_ms": {n: round(kms[n], 4) for n in path_kernels},
                    "segments": {"chunks_first_segment": l0, "chunks_per_segment": lseg, "segments_per_head": ns}},
        "mfma": mfma,
        # ms_per_step: events around each call (the event records' own cost included);
        # kernel_*: the decode kernel's average duration from the library's timing
        "decode": {"ms_per_step": dst, "GBps": round(dec_gbs, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "tokens_per_s": round(DEC_N / (dec_ms * 1e-3), 1),
                   "kernel_ms": round(kms["decode"], 4),
                   "kernel_GBps": round(DEC_N * DEC_H * DECODE_BYTES_PER_HEAD / (kms["decode"] * 1e-3) / 1e9, 1),
                   "kernel_hbm_frac": round(DEC_N * DEC_H * DECODE_BYTES_PER_HEAD / (kms["decode"] * 1e-3) / 1e9
                                            / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "kernels": kernels,
        "kernel_source_hash": src_hash,
    }
    extras = set() if args.no_extras else {x for x in args.extras.split(",") if x}
    if args.no_backward:
        extras.discard("backward")
    if args.no_dplr:
        extras.discard("dplr")
    if "configs" in extras:
        result["configs"] = config_timing(inputs, kda, torch, dev)
    if "paths" in extras:
        result["paths"] = path_timing(kda, torch, pre)
    if "fused" in extras:
        result["fused"] = fused_timing(inputs, kda, torch, dev, pre, dec, state, o_dec)
    if "gates" in extras:
        result["gates"] = gate_timing(kda, torch, pre, dec, state, o_dec)
    if "backward" in extras:
        del ws
        torch.cuda.empty_cache()
        result["backward"] = backward_timing(inputs, kda, torch, pre)
    if "dplr" in extras:
        lengths = tuple(int(x) for x in args.dplr_lengths.split(",") if x)
        result["dplr_comparison"] = dplr_comparison(inputs, kda, torch, dev, pre, lengths=lengths)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        base, threads = cpu_baselines(inputs, pre, dec)
        head = base["kda_prefill_T131072_H32_bf16"]
        result["cpu_baseline"] = {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"all {head['tokens']} tokens x {head['heads']} heads of the headline "
                                            f"prefill workload (fp64 sequential recurrence, {head['seconds']} s)",
                                  "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
        result["cpu_baselines"] = base
    result["environment"] = environment(torch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
