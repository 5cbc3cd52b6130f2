"""Host logic of the profile summaries: kernel-name shortening and the counter
scaling that turns FETCH_SIZE / WRITE_SIZE readings into bytes per launch."""
import csv
import os

from gated_delta_rule_57_amd import profiling


def test_short_names_split_intra_by_gate():
    s = profiling.short_name
    assert s("_ZN3kda12intra_kernelIDF16bLi64ELi0EEEvPKT_S3_") == "intra"
    assert s("_ZN3kda12intra_kernelIDF16bLi64ELi1EEEvPKT_S3_") == "intra_gdn"
    assert s("_ZN3kda12intra_kernelIfLi64ELi2EEEvPKT_S3_") == "intra_deltanet"
    assert s("_ZN3kda12intra_kernelIfLi16ELi2EEEvPKT_S3_") == "intra_deltanet16"
    assert s("void kda::intra_kernel<__bf16, 64, 1>(__bf16 const*)") == "intra_gdn"
    assert s("void kda::inter_wg_kernel<1>(char const*, int const*)") == "inter"
    assert s("_ZN3kda13decode_kernelIDF16bEEvPKT_") == "decode"
    assert s("_ZN3kda23output_norm_gate_kernelIDF16bEEvPKT_") == "outnorm"
    assert s("kda::plan_kernel(int const*, int)") == "plan"
    assert s("__amd_rocclr_copyBuffer") is None
    assert s("_ZN3kda12intra_kernelIDF16bLi16ELi0EEEvPKT_S3_") == "intra16"
    assert s("void kda::intra_kernel<__bf16, 16, 0>(__bf16 const*)") == "intra16"
    assert s("void kda::inter16_kernel<__bf16>(char const*, int const*)") == "inter16"
    assert s("_ZN3kda12_GLOBAL__N_116bwd_chunk_kernelIDF16bEEvPKT_") == "bwd_chunk"
    assert s("_ZN3kda12_GLOBAL__N_116bwd_state_kernelIDF16bEEvPKc") == "bwd_state"
    assert s("_ZN3kda12_GLOBAL__N_116fwd_state_kernelIDF16bEEvPKc") == "inter16"
    assert s("_ZN3kda15inter_wg_kernelILi1ELb0EEEvPKcPKiS4_iiPKfPfPDF16biii") == "inter"
    assert s("_ZN3kda15inter_wg_kernelILi1ELb1EEEvPKcPKiS4_iiPKfPfPDF16biii") == "dplr_inter"
    assert s("_ZN3kda12inter_kernelIfLi64ELb1EEEvPKcPKiPK15HIP_vector_typeIiLj2EE") == "dplr_inter"
    assert s("_ZN3kda12inter_kernelIfLi64ELb0EEEvPKcPKiPK15HIP_vector_typeIiLj2EE") == "inter"
    assert s("void kda::inter_wg_kernel<1, true>(char const*)") == "dplr_inter"
    assert s("_ZN3kda17dplr_intra_kernelIDF16bEEvPKT_S3_S3_S3_S3_PKfPKiPK15HIP_vector_typeIiLj2EEiiPc") == "dplr_intra"
    assert s("_ZN3kda12_GLOBAL__N_116bwd_local_kernelIDF16bEEvPKT_") == "bwd_local"


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_traffic_scaling(tmp_path):
    root = str(tmp_path)
    gib_kib = (1 << 30) / 1024
    # the copy of 1 GiB reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _write_counters(os.path.join(root, "copy_FETCH_SIZE"), [["__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2]])
    _write_counters(os.path.join(root, "copy_WRITE_SIZE"), [["__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib]])
    _write_counters(os.path.join(root, "bench_FETCH_SIZE"), [["kda::plan_kernel(int)", "FETCH_SIZE", 10.0],
                                                            ["kda::plan_kernel(int)", "FETCH_SIZE", 30.0]])
    _write_counters(os.path.join(root, "bench_WRITE_SIZE"), [["kda::plan_kernel(int)", "WRITE_SIZE", 4.0]])
    out = os.path.join(root, "t.json")
    profiling.summarize_traffic(root, out, "cmd")
    import json
    d = json.load(open(out))
    assert abs(d["calibration"]["FETCH_SIZE"]["scale"] - 2.0) < 1e-12
    assert d["kernels"]["plan"]["fetch_size_bytes_scaled"] == 20.0 * 1024 * 2
    assert d["kernels"]["plan"]["write_size_bytes_scaled"] == 4.0 * 1024
    assert d["kernels"]["plan"]["hbm_bytes_per_launch"] == 20.0 * 1024 * 2 + 4.0 * 1024


def test_bench_backward_byte_counts_match_the_workspace_layout():
    """The per-(chunk, head) sizes behind bench.py's backward byte counts (forward
    record 22016 B; backward record, two 128 x 128 bf16 matrices, two 16 x 128 ones
    and the fp32 16 x 16 T and M, 89088 B) agree with the library's workspace queries."""
    import bench
    from gated_delta_rule_57_amd import kda
    T, H = 4096, 16
    mc = T // bench.BWD_CHUNK
    fwd = kda.workspace_size(1, T, H, chunk=16)
    bwd = kda.bwd_workspace_size(1, T, H)
    assert abs(fwd / (mc * H) - 22016) < 1
    assert (bwd - fwd) == mc * H * (13312 + 2 * 32768 + 2 * 4096 + bench.BWD_TM_BYTES)


def test_bench_record_byte_counts_match_the_workspace_queries():
    """The per-(64-token chunk, head) record sizes behind bench.py's KDA and DPLR
    byte counts agree with the library's workspace queries."""
    import bench
    from gated_delta_rule_57_amd import kda
    T, H = 4096, 16
    mc = T // bench.CHUNK
    assert abs(kda.workspace_size(1, T, H, chunk=64, path="record") / (mc * H) - bench.RECORD_BYTES_BF16_C64) < 1
    assert abs(kda.dplr_workspace_size(1, T, H) / (mc * H) - bench.DPLR_RECORD_BYTES_BF16) < 1


def test_short_names_of_the_segment_parallel_kernels():
    s = profiling.short_name
    assert s("_ZN3kda15seg_plan_kernelEPKiiiiiiPiP15HIP_vector_typeIiLj2EE") == "seg_plan"
    assert s("_ZN3kda15seg_scan_kernelEPKiiiPfS2_") == "seg_scan"
    assert s("_ZN3kda14rec_seg_kernelILb0EEEvNS_7SegArgsE") == "seg_first"
    assert s("_ZN3kda14rec_seg_kernelILb1EEEvNS_7SegArgsE") == "seg_second"
    assert s("void kda::rec_seg_kernel<true>(kda::SegArgs)") == "seg_second"
    assert s("_ZN3kda15seg_pass_kernelILi0ELb0EEEvNS_7SegArgsE") == "single_first"
    assert s("_ZN3kda15seg_pass_kernelILi0ELb1EEEvNS_7SegArgsE") == "single_second"
    assert s("void kda::seg_pass_kernel<1, false>(kda::SegArgs)") == "single_first"
    # with the output-epilogue flag after the pass flag
    assert s("_ZN3kda12_GLOBAL__N_114rec_seg_kernelILb1ELb0EEEvNS0_7SegArgsE") == "seg_second"
    assert s("_ZN3kda12_GLOBAL__N_114rec_seg_kernelILb0ELb1EEEvNS0_7SegArgsE") == "seg_first_gated"
    assert s("void kda::(anonymous namespace)::rec_seg_kernel<false, false>(kda::SegArgs)") == "seg_first"
    assert s("void kda::(anonymous namespace)::rec_seg_kernel<true, true>(kda::SegArgs)") == "seg_second_gated"
    assert s("_ZN3kda12_GLOBAL__N_115seg_pass_kernelILi0ELb1ELb0EEEvNS0_7SegArgsE") == "single_second"
    assert s("_ZN3kda12_GLOBAL__N_115seg_pass_kernelILi2ELb0ELb1EEEvNS0_7SegArgsE") == "single_first_gated"
    assert s("void kda::(anonymous namespace)::seg_pass_kernel<0, true, true>(kda::SegArgs)") == "single_second_gated"


def test_bench_segment_plan_matches_the_workspace_query():
    """bench.py's copy of the segment plan (a shorter first segment, then segments of
    lseg chunks) gives the segment count the library sizes its segmented workspace
    for (per-segment maps and entry states), for both kernel sets: room for the plan
    with the output epilogue and the one without."""
    import bench
    from gated_delta_rule_57_amd import kda
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    st = 128 * 128 * 4
    for T, H in ((131072, 32), (4096, 16), (32768, 32), (64 * 40 + 37, 2), (64, 4)):
        for kernels, path in (("record", "segmented"), ("single", "single")):
            nc = (T + 63) // 64
            seg = 0
            for gated in (False, True):
                lseg, l0, ns = bench.seg_plan(T, H, kernels=kernels, gated=gated)
                assert 1 <= l0 <= lseg and (ns == 1 or l0 + (ns - 2) * lseg < nc <= l0 + (ns - 1) * lseg)
                seg = max(seg, al(2 * 4) + al(ns * 8) + al(ns * H * st) + al(ns * H * 2 * st))
            rec = al(kda.workspace_size(1, T, H, chunk=64, path="record")) if path == "segmented" else 0
            assert kda.workspace_size(1, T, H, chunk=64, path=path) - rec == seg, (T, H, kernels)
    assert bench.seg_plan(131072, 32) == (240, 132, 9)
    assert bench.seg_plan(131072, 32, gated=True) == (244, 103, 9)


def test_mfma_summary(tmp_path):
    """Counted MFMA flops (512 per MOPS unit) over the traced average duration,
    against 2.5 PFLOP/s bf16 and 157.3 TFLOP/s fp32."""
    import json
    root = str(tmp_path)
    name = "_ZN3kda12intra_kernelIDF16bLi64ELi0EEEvPKT_S3_"
    _write_counters(os.path.join(root, "bench_SQ_INSTS_VALU_MFMA_MOPS_BF16"),
                    [[name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.5e6], [name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 7.5e6]])
    _write_counters(os.path.join(root, "bench_SQ_INSTS_VALU_MFMA_MOPS_F32"), [[name, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0]])
    _write_counters(os.path.join(root, "bench_SQ_VALU_MFMA_BUSY_CYCLES"), [[name, "SQ_VALU_MFMA_BUSY_CYCLES", 30.0]])
    _write_counters(os.path.join(root, "bench_SQ_BUSY_CU_CYCLES"), [[name, "SQ_BUSY_CU_CYCLES", 120.0]])
    trace = os.path.join(root, "trace")
    os.makedirs(trace)
    with open(os.path.join(trace, "x_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow([name, 2, 2.0e6, 1.0e6, 100.0, 1.0e6, 1.0e6])
    out = os.path.join(root, "m.json")
    profiling.summarize_mfma(root, trace, out, "cmd")
    d = json.load(open(out))
    k = d["kernels"]["intra"]
    assert k["mfma_flops_bf16"] == 5.0e6 * 512
    assert abs(k["mfma_util"] - 5.0e6 * 512 / 1e-3 / 2.5e15) < 1e-12
    assert abs(k["mfma_busy_over_cu_busy"] - 0.25) < 1e-12
    assert d["summary"]["prefill_kernels"] == ["intra"]


def test_mfma_summary_reads_the_derived_busy_counter(tmp_path):
    import json
    root = str(tmp_path)
    name = "_ZN3kda14rec_seg_kernelILb1EEEvNS_7SegArgsE"
    _write_counters(os.path.join(root, "bench_MfmaUtil"), [[name, "MfmaUtil", 12.0], [name, "MfmaUtil", 14.0]])
    _write_counters(os.path.join(root, "bench_SQ_INSTS_VALU_MFMA_MOPS_BF16"),
                    [[name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1.0e6], [name, "SQ_INSTS_VALU_MFMA_MOPS_F32", 1.0e5]])
    trace = os.path.join(root, "trace")
    os.makedirs(trace)
    with open(os.path.join(trace, "x_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow([name, 1, 5.0e5, 5.0e5, 100.0, 5.0e5, 5.0e5])
    out = os.path.join(root, "m.json")
    profiling.summarize_mfma(root, trace, out, "cmd")
    d = json.load(open(out))
    k = d["kernels"]["seg_second"]
    assert abs(k["mfma_busy"] - 0.13) < 1e-12
    want = 1.0e6 * 512 / 5e-4 / 2.5e15 + 1.0e5 * 512 / 5e-4 / 157.3e12
    assert abs(k["mfma_util"] - want) < 1e-12
    assert d["summary"]["prefill_mfma_busy"] == 0.13
