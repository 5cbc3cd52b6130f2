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
    record 22016 B; backward record, two 128 x 128 bf16 matrices and two 16 x 128
    ones 87040 B) agree with the library's workspace queries."""
    import bench
    from gated_delta_rule_57_amd import kda
    T, H = 4096, 16
    mc = T // bench.BWD_CHUNK
    fwd = kda.workspace_size(1, T, H, chunk=16)
    bwd = kda.bwd_workspace_size(1, T, H)
    assert abs(fwd / (mc * H) - 22016) < 1
    assert (bwd - fwd) == mc * H * (13312 + 2 * 32768 + 2 * 4096)


def test_bench_record_byte_counts_match_the_workspace_queries():
    """The per-(64-token chunk, head) record sizes behind bench.py's KDA and DPLR
    byte counts agree with the library's workspace queries."""
    import bench
    from gated_delta_rule_57_amd import kda
    T, H = 4096, 16
    mc = T // bench.CHUNK
    assert abs(kda.workspace_size(1, T, H, chunk=64) / (mc * H) - bench.RECORD_BYTES_BF16_C64) < 1
    assert abs(kda.dplr_workspace_size(1, T, H) / (mc * H) - bench.DPLR_RECORD_BYTES_BF16) < 1
