"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill over a 131072-token sequence with 32 heads of
dimension 128 (bf16 q/k/v, fp32 decays and state, chunk 64), followed by
``--decode-per-step`` decode steps over 256 sequences x 32 heads of persisted fp32
128 x 128 states (bf16 q/k/v). Inputs are synthetic, seeded and resident in HBM
before timing starts.

Prints one JSON line. ``value`` is prefill tokens/s (a token = one position across
all 32 heads), from HIP events recorded by the library on the stream its kernels
run on. Decode throughput (GB/s of state + vectors, fraction of HBM peak), the
algorithmic fraction of bf16 MFMA peak, per-kernel roofline figures and the CPU
oracle's throughput on a sample of the same workload are reported beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA

D = 128
CHUNK = 64
# algorithmic flops per (token, head) of the chunked prefill at C = 64, d = 128 (triangles
# counted exactly): state products 6 d^2, A (C-1) d, P (C+1) d, P U~ (C+1) d, T [bK | bV] (C-1) 2d
FLOP_PER_TOK_HEAD = 6 * D * D + (CHUNK - 1) * D + (CHUNK + 1) * D + (CHUNK + 1) * D + (CHUNK - 1) * 2 * D
# bytes every prefill must move per (token, head): q, k, v bf16, log_alpha fp32, beta fp32, o bf16
PATH_BYTES_PER_TOK_HEAD = 3 * 2 * D + 4 * D + 4 + 2 * D
# per-(chunk, head) record written by the intra-chunk kernel and read by the inter-chunk kernel:
# its size in the workspace, and the bytes actually moved (the two all-zero P slots above the
# diagonal, 2 x 1 KiB, are neither written nor read)
RECORD_BYTES_BF16_C64 = 74240
RECORD_MOVED_BYTES_BF16_C64 = RECORD_BYTES_BF16_C64 - 2048
# one decode (sequence, head): fp32 state read + written, q, k, v bf16, log_alpha fp32, beta, o bf16
DECODE_BYTES_PER_HEAD = 2 * 4 * D * D + 3 * 2 * D + 4 * D + 4 + 2 * D

# backward (16-token chunks, bf16): per (chunk, head) the forward record (22016 B), the
# backward record (13312 B), the chunk-entry state and the chunk-end state gradient
# (2 x 32768 B) and U~, dU~ (2 x 4096 B); per (token, head) algorithmic bytes of each kernel
BWD_CHUNK = 16
BWD_BYTES_PER_TOK_HEAD = {
    "intra": 3 * 2 * D + 4 * D + 4 + 22016 // BWD_CHUNK,                    # inputs in, record out
    "inter": 22016 // BWD_CHUNK + (32768 + 4096) // BWD_CHUNK,              # record in, states and U~ out
    "bwd_local": 2 * 2 * D + 4 * D + 4 + 13312 // BWD_CHUNK,                # q, k, gate in, record out
    "bwd_state": 13312 // BWD_CHUNK + 2 * D + (32768 + 4096) // BWD_CHUNK,  # record, grad_o in, dS_C, dU~ out
    "bwd_chunk": 4 * 2 * D + 4 * D + 4 + 2 * (32768 + 4096) // BWD_CHUNK + 3 * 2 * D + 4 * D + 4,
}
# bytes any backward must move per (token, head): q, k, v, grad_o, log_alpha, beta in; the five gradients out
BWD_PATH_BYTES_PER_TOK_HEAD = 4 * 2 * D + 4 * D + 4 + 3 * 2 * D + 4 * D + 4

# general DPLR forward (64-token chunks, bf16): per (chunk, head) record of 123392 B
DPLR_RECORD_BYTES_BF16 = 123392
DPLR_RECORD_MOVED_BYTES_BF16 = DPLR_RECORD_BYTES_BF16 - 2048
DPLR_IN_BYTES_PER_TOK_HEAD = 5 * 2 * D + 4 * D   # q, k, v, a, b bf16, log_alpha fp32

PREFILL_T, PREFILL_H = 131072, 32
DEC_N, DEC_H = 256, 32


def kernel_source_hash():
    from gated_delta_rule_57_amd.profiling import kernel_source_hash as source_hash
    return source_hash(ROOT)


def traffic_from_profiles(kernel, src_hash):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_hash") != src_hash:
        return None
    ent = data.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(inp, sample_tokens):
    """The fp64 sequential oracle on the first ``sample_tokens`` tokens of the same
    prefill workload (all heads), on this host's cores."""
    import numpy as np
    import oracle

    S = min(sample_tokens, inp.q.shape[1])
    f = lambda t: t[:, :S].float().cpu().numpy()
    q, k, v, la, beta = f(inp.q), f(inp.k), f(inp.v), f(inp.log_alpha), f(inp.beta)
    threads = oracle.seq.default_threads()
    t0 = time.perf_counter()
    o, fin = oracle.forward(q, k, v, la, beta, num_threads=threads)
    dt = time.perf_counter() - t0
    assert np.isfinite(o).all()
    return {"value": S / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {inp.q.shape[1]} tokens of the prefill workload, all {inp.q.shape[2]} heads "
                      f"(fp64 sequential recurrence, {dt:.1f} s)"}


def fused_timing(inputs, kda, torch, dev, pre, dec, ws, o, fin, state, o_dec, runs=5):
    """The fused layer core on the same shapes: the prefill on raw q, k and gate /
    beta pre-activations with the output RMSNorm and gate, and the fused decode
    step. Timed by the library's events, outside the headline steps."""
    B, T, H = pre.q.shape[:3]
    raw = inputs.make_raw_prefill(3, B=B, T=T, H=H, dtype="bf16", device=dev)
    fu = kda.fusion(out_gate=raw.out_gate, norm_weight=raw.norm_weight)
    z_dec = torch.randn(o_dec.shape, device=dev).to(o_dec.dtype)
    fu_dec = kda.fusion(out_gate=z_dec, norm_weight=raw.norm_weight)

    def prefill():
        kda.chunk_fwd(raw.q, raw.k, raw.v, raw.gate, raw.beta, chunk=CHUNK, o=o, final_state=fin, workspace=ws,
                      fusion=fu)

    def decode(i):
        kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], state, o=o_dec, fusion=fu_dec)

    for i in range(2):
        prefill()
        decode(i)
    torch.cuda.synchronize()
    kda.timing_enable(True)
    for i in range(runs):
        prefill()
        for j in range(8):
            decode((i * 8 + j) % dec.q.shape[0])
    torch.cuda.synchronize()
    t = kda.timing_read()
    kda.timing_enable(False)
    ms = {name: tot / max(cnt, 1) for name, (tot, cnt) in t.items()}
    prefill_ms = ms["plan"] + ms["intra"] + ms["inter"] + ms["outnorm"]
    rows = T * H
    outnorm_bytes = rows * 3 * 2 * D + 4 * D
    dec_bytes = DEC_N * DEC_H * (DECODE_BYTES_PER_HEAD + 2 * D)
    print(f"[bench] fused prefill {prefill_ms:.3f} ms", file=sys.stderr, flush=True)
    return {"workload": "kda_prefill_T131072_H32_bf16 raw inputs (q, k unnormalised; gate and beta "
                        "pre-activations; output RMSNorm and sigmoid gate) + kda_decode_N256_H32_bf16",
            "prefill_ms": round(prefill_ms, 4), "tokens_per_s": round(T / (prefill_ms * 1e-3), 1),
            "kernel_ms": {k: round(ms[k], 4) for k in ("plan", "intra", "inter", "outnorm")},
            "outnorm_GBps": round(outnorm_bytes / (ms["outnorm"] * 1e-3) / 1e9, 1),
            "decode_ms_per_step": round(ms["decode"], 4),
            "decode_GBps": round(dec_bytes / (ms["decode"] * 1e-3) / 1e9, 1)}


def backward_timing(inputs, kda, torch, pre, runs=3):
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
    kda.timing_enable(True)
    for _ in range(runs):
        g = run()
    torch.cuda.synchronize()
    t = kda.timing_read()
    kda.timing_enable(False)
    ms = {n: tot / max(cnt, 1) for n, (tot, cnt) in t.items() if cnt}
    names = ("plan", "intra", "inter", "bwd_local", "bwd_state", "bwd_chunk")
    total = sum(ms.get(n, 0.0) for n in names)
    tok_heads = T * H
    gbps = {n: round(BWD_BYTES_PER_TOK_HEAD[n] * tok_heads / (ms[n] * 1e-3) / 1e9, 1)
            for n in names if n in BWD_BYTES_PER_TOK_HEAD}
    finite = all(bool(torch.isfinite(x).all()) for x in g.values() if x is not None)
    del g, ws, grad_o
    torch.cuda.empty_cache()
    print(f"[bench] backward {total:.3f} ms", file=sys.stderr, flush=True)
    return {"workload": "kda_backward_T131072_H32_bf16 (gradients of q, k, v, log_alpha, beta and the initial "
                        "state; 16-token chunks)",
            "ms": round(total, 4), "tokens_per_s": round(T / (total * 1e-3), 1),
            "kernel_ms": {n: round(ms.get(n, 0.0), 4) for n in names},
            "kernel_GBps_algorithmic": gbps,
            "path_hbm_frac_ideal": round(BWD_PATH_BYTES_PER_TOK_HEAD * tok_heads / (total * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
            "finite": finite}


def gate_timing(kda, torch, pre, dec, ws, o, fin, state, o_dec, runs=5):
    """The scalar-gate (one decay per token and head) and no-decay paths on the
    headline prefill shape and the decode batch, timed by the library's events."""
    B, T, H = pre.q.shape[:3]
    la_head = pre.log_alpha[..., 0].contiguous()
    la_dec = dec.log_alpha[..., 0].contiguous()
    out = {}
    for name, la, lad in (("gated_deltanet", la_head, la_dec), ("deltanet", None, None)):
        def run(i):
            kda.chunk_fwd(pre.q, pre.k, pre.v, la, pre.beta, chunk=CHUNK, o=o, final_state=fin, workspace=ws)
            for j in range(8):
                d = (i * 8 + j) % dec.q.shape[0]
                kda.decode_step(dec.q[d], dec.k[d], dec.v[d], None if lad is None else lad[d], dec.beta[d], state,
                                o=o_dec)
        run(0)
        torch.cuda.synchronize()
        kda.timing_enable(True)
        for i in range(runs):
            run(i + 1)
        torch.cuda.synchronize()
        t = kda.timing_read()
        kda.timing_enable(False)
        ms = {n: tot / max(cnt, 1) for n, (tot, cnt) in t.items()}
        prefill_ms = ms["plan"] + ms["intra"] + ms["inter"]
        tok_heads = T * H
        gate_bytes = 0 if la is None else 4
        intra_bytes = tok_heads * (3 * 2 * D + gate_bytes + 4) + (T // CHUNK) * H * RECORD_MOVED_BYTES_BF16_C64
        out[name] = {"prefill_ms": round(prefill_ms, 4), "tokens_per_s": round(T / (prefill_ms * 1e-3), 1),
                     "kernel_ms": {k: round(ms[k], 4) for k in ("plan", "intra", "inter")},
                     "intra_GBps": round(intra_bytes / (ms["intra"] * 1e-3) / 1e9, 1),
                     "decode_ms_per_step": round(ms["decode"], 4)}
        print(f"[bench] {name} prefill {prefill_ms:.3f} ms", file=sys.stderr, flush=True)
    return out


def dplr_comparison(inputs, kda, torch, dev, pre, ws, lengths=(4096, 16384, 65536, 131072), runs=3):
    """KDA's chunked forward against the general DPLR chunked forward
    (kda_dplr_chunk_fwd) on the same shapes: H = 32, d = 128, bf16, 64-token chunks,
    over input lengths. Prefixes of one 131072-token input set per method (KDA: the
    headline workload; DPLR: the stable tied recipe with the same mixed decays).
    Times are the library's per-kernel events (plan + intra + inter)."""
    B, Tmax, H = pre.q.shape[:3]
    x = inputs.make_dplr(3, B=1, T=Tmax, H=H, dtype="bf16", la_mode="mixed", device=dev)
    ws_d = torch.empty(kda.dplr_workspace_size(1, Tmax, H, 0, kda.KDA_BF16), dtype=torch.uint8, device=dev)
    o = torch.empty_like(pre.v)
    fin = torch.empty(1, H, D, D, dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        kda.timing_enable(True)
        for _ in range(runs):
            fn()
        torch.cuda.synchronize()
        t = kda.timing_read()
        kda.timing_enable(False)
        ms = {n: tot / max(cnt, 1) for n, (tot, cnt) in t.items() if cnt}
        return {n: ms.get(n, 0.0) for n in ("plan", "intra", "inter")}

    rows = []
    for T in lengths:
        if T > Tmax:
            continue
        sl = lambda t: t[:, :T]
        km = timed(lambda: kda.chunk_fwd(sl(pre.q), sl(pre.k), sl(pre.v), sl(pre.log_alpha), sl(pre.beta),
                                         chunk=CHUNK, o=o[:, :T], final_state=fin, workspace=ws))
        dm = timed(lambda: kda.dplr_chunk_fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.a), sl(x.b), sl(x.log_alpha),
                                              o=o[:, :T], final_state=fin, workspace=ws_d))
        kt, dt = sum(km.values()), sum(dm.values())
        tok_heads = T * H
        d_intra_bytes = tok_heads * DPLR_IN_BYTES_PER_TOK_HEAD + (T // CHUNK) * H * DPLR_RECORD_MOVED_BYTES_BF16
        d_inter_bytes = (T // CHUNK) * H * DPLR_RECORD_MOVED_BYTES_BF16 + tok_heads * 2 * D
        rows.append({"T": T, "kda_ms": round(kt, 4), "dplr_ms": round(dt, 4),
                     "dplr_over_kda": round(dt / kt, 3),
                     "kda_tokens_per_s": round(T / (kt * 1e-3), 1), "dplr_tokens_per_s": round(T / (dt * 1e-3), 1),
                     "kda_kernel_ms": {n: round(v, 4) for n, v in km.items()},
                     "dplr_kernel_ms": {n: round(v, 4) for n, v in dm.items()},
                     "dplr_intra_GBps": round(d_intra_bytes / (dm["intra"] * 1e-3) / 1e9, 1),
                     "dplr_inter_GBps": round(d_inter_bytes / (dm["inter"] * 1e-3) / 1e9, 1)})
        print(f"[bench] T={T}: kda {kt:.3f} ms, dplr {dt:.3f} ms ({dt / kt:.2f}x)", file=sys.stderr, flush=True)
    del x, ws_d, o, fin
    torch.cuda.empty_cache()
    return {"workload": "kda_vs_dplr_H32_bf16_c64 (prefill at several lengths; the general DPLR transition "
                        "Diag(alpha) + a b^T with free a, b against KDA's key-tied one)",
            "lengths": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-per-step", type=int, default=8)
    ap.add_argument("--decode-inputs", type=int, default=1024, help="distinct decode tokens, cycled")
    ap.add_argument("--cpu-sample-tokens", type=int, default=PREFILL_T)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gates", action="store_true",
                    help="skip the timing of the scalar-gate (Gated DeltaNet) and no-decay (DeltaNet) paths")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the timing of the fused layer core (prologue and epilogue in the kernels)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the backward (kda_chunk_bwd) on the prefill shape")
    ap.add_argument("--no-dplr", action="store_true",
                    help="skip the KDA versus general-DPLR forward comparison over input lengths")
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
    ws = torch.empty(kda.workspace_size(B, T, H, 0, CHUNK, kda.KDA_BF16), dtype=torch.uint8, device=dev)
    o = torch.empty_like(pre.v)
    fin = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    state = dec.initial_state.clone()
    o_dec = torch.empty(DEC_N, DEC_H, D, dtype=torch.bfloat16, device=dev)
    n_dec_in = dec.q.shape[0]
    dec_i = [0]

    def step():
        kda.chunk_fwd(pre.q, pre.k, pre.v, pre.log_alpha, pre.beta, chunk=CHUNK, o=o, final_state=fin,
                      workspace=ws)
        for _ in range(args.decode_per_step):
            i = dec_i[0] % n_dec_in
            kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], state, o=o_dec)
            dec_i[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    kda.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timing = kda.timing_read()
    kda.timing_enable(False)
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    K = args.steps
    ms = {name: tot / max(cnt, 1) for name, (tot, cnt) in timing.items()}
    prefill_ms = ms["plan"] + ms["intra"] + ms["inter"]
    tokens_per_s = T / (prefill_ms * 1e-3)
    tok_heads = T * H
    flops = FLOP_PER_TOK_HEAD * tok_heads
    prefill_tflops = flops / (prefill_ms * 1e-3) / 1e12
    n_chunks = (T + CHUNK - 1) // CHUNK
    rec_bytes = n_chunks * H * RECORD_MOVED_BYTES_BF16_C64
    in_bytes = tok_heads * (3 * 2 * D + 4 * D + 4)
    out_bytes = tok_heads * 2 * D
    kernel_bytes = {
        "intra": in_bytes + rec_bytes,            # reads the chunk's inputs, writes its record
        "inter": rec_bytes + out_bytes,            # reads the records once per head, writes o
        "decode": DEC_N * DEC_H * DECODE_BYTES_PER_HEAD,
    }
    src_hash = kernel_source_hash()
    kernels = {}
    for name in ("intra", "inter", "decode"):
        t_s = ms[name] * 1e-3
        gbs = kernel_bytes[name] / t_s / 1e9
        traffic = traffic_from_profiles(name, src_hash)
        kernels[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "avg_ms": round(ms[name], 4), "launches": timing[name][1],
                         "algorithmic_bytes_per_launch": kernel_bytes[name]}
    per_step = {"intra": ms["intra"], "inter": ms["inter"], "decode": ms["decode"] * args.decode_per_step}
    dominant = max(per_step, key=per_step.get)
    roof = {k: kernels[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dominant
    dec_gbs = kernel_bytes["decode"] / (ms["decode"] * 1e-3) / 1e9

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
                   "parallelism": "single GPU"},
        "prefill": {"ms": round(prefill_ms, 4), "tokens_per_s": round(tokens_per_s, 1),
                    "algorithmic_tflops": round(prefill_tflops, 2),
                    "mfma_frac_algorithmic": round(prefill_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                    "path_hbm_frac_ideal": round(PATH_BYTES_PER_TOK_HEAD * tok_heads / (prefill_ms * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 4),
                    "kernel_ms": {"plan": round(ms["plan"], 4), "intra": round(ms["intra"], 4),
                                  "inter": round(ms["inter"], 4)}},
        "decode": {"ms_per_step": round(ms["decode"], 4), "GBps": round(dec_gbs, 1),
                   "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "tokens_per_s": round(DEC_N / (ms["decode"] * 1e-3), 1)},
        "roofline": roof,
        "kernels": kernels,
        "kernel_source_hash": src_hash,
    }
    if not args.no_fused:
        result["fused"] = fused_timing(inputs, kda, torch, dev, pre, dec, ws, o, fin, state, o_dec)
    if not args.no_gates:
        result["gates"] = gate_timing(kda, torch, pre, dec, ws, o, fin, state, o_dec)
    if not args.no_backward:
        result["backward"] = backward_timing(inputs, kda, torch, pre)
    if not args.no_dplr:
        lengths = tuple(int(x) for x in args.dplr_lengths.split(",") if x)
        result["dplr_comparison"] = dplr_comparison(inputs, kda, torch, dev, pre, ws, lengths=lengths)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pre, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
