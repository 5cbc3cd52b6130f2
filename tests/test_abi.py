"""The C ABI of libkda.so on the CPU: the library loads, exports every entry point
include/kda.h declares, and every invalid argument is rejected with its status
before any HIP call is made (so none of these tests touches a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

from gated_delta_rule_57_amd import kda  # noqa: E402  (loads libkda.so; fails loudly if missing)

L = kda.lib
FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced by the host checks
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_symbol():
    for name in header_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    version = int(re.search(r"#define KDA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.kda_abi_version() == version == 5
    for st in (0, -1, -2, -3, -4):
        assert L.kda_status_string(st).decode().startswith("KDA_")
    assert b"unknown" in L.kda_status_string(7)


def chunk_call(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, s0=None, cu=None, num_seqs=0, o=FAKE, fin=FAKE,
               B=1, T=64, H=2, dk=128, dv=128, chunk=64, dtype=0, ws=None, ws_bytes=0):
    return L.kda_chunk_fwd(q, k, v, la, beta, s0, cu, num_seqs, o, fin, B, T, H, dk, dv, chunk, dtype, ws,
                           ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=0), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=5), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(B=-2), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(k=None), kda.KDA_ERR_INVALID_ARG),
    (dict(v=None), kda.KDA_ERR_INVALID_ARG),
    (dict(la=None), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(q=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(fin=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(s0=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=ctypes.c_void_p((1 << 20) + 2)), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=2, B=2), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=0, T=10), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=ctypes.c_void_p((1 << 20) + 2), num_seqs=2), kda.KDA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=1 << 30), kda.KDA_ERR_INVALID_ARG),
    (dict(ws=FAKE, ws_bytes=16), kda.KDA_ERR_WORKSPACE),
    (dict(B=1 << 16, T=1 << 16), kda.KDA_ERR_INVALID_ARG),
    # 2^26 chunks of 16 tokens times 64 heads: more (chunk, head) work-groups than a 1-D grid holds
    (dict(T=1 << 30, H=64, chunk=16), kda.KDA_ERR_INVALID_ARG),
])
def test_chunk_fwd_rejects(kw, status):
    assert chunk_call(**kw) == status
    assert L.kda_last_error().decode() != ""


def test_chunk_fwd_empty_batch_is_ok_without_device():
    assert chunk_call(B=0, q=None, k=None, v=None, la=None, beta=None, o=None, fin=None) == kda.KDA_OK
    assert L.kda_last_error().decode() == ""
    assert chunk_call(cu=FAKE, num_seqs=0, T=0) == kda.KDA_OK


def decode_call(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, state=FAKE, o=FAKE, N=4, H=2, dk=128, dv=128, dtype=0):
    return L.kda_decode_step(q, k, v, la, beta, state, o, N, H, dk, dv, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=-1), kda.KDA_ERR_UNSUPPORTED),
    (dict(N=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(state=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=ctypes.c_void_p((1 << 20) + 2)), kda.KDA_ERR_INVALID_ARG),
    (dict(state=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
])
def test_decode_rejects(kw, status):
    assert decode_call(**kw) == status


def test_decode_empty_batch_is_ok():
    assert decode_call(N=0, q=None, state=None) == kda.KDA_OK


def path_ws(path, B, T, H, num_seqs, chunk, dtype):
    f = kda.Fusion()
    f.prefill_path = path
    return L.kda_chunk_fwd_fused_workspace_size(B, T, H, num_seqs, chunk, dtype, ctypes.byref(f))


def record_ws(*args):
    return path_ws(kda.KDA_PATH_RECORD, *args)


def single_ws(*args):
    return path_ws(kda.KDA_PATH_SINGLE_PASS, *args)


def test_workspace_size():
    ws = L.kda_chunk_fwd_workspace_size
    assert ws(1, 64, 1, 0, 16, 1) > 0
    # the record paths hold one record per (chunk, head): they grow with tokens and heads
    assert record_ws(1, 4096, 16, 0, 64, 0) < record_ws(1, 8192, 16, 0, 64, 0) < record_ws(1, 8192, 32, 0, 64, 0)
    assert record_ws(1, 4096, 16, 0, 64, 0) < record_ws(1, 4096, 16, 0, 64, 1)
    # fp32 and 16-token chunks have one path; every path value gives its size
    for path in (kda.KDA_PATH_AUTO, kda.KDA_PATH_RECORD, kda.KDA_PATH_SINGLE_PASS, kda.KDA_PATH_RECORD_SEGMENTED):
        assert path_ws(path, 1, 4096, 16, 0, 64, 1) == record_ws(1, 4096, 16, 0, 64, 1)
        assert path_ws(path, 1, 4096, 16, 0, 16, 0) == record_ws(1, 4096, 16, 0, 16, 0)
    # bf16, 64-token chunks: the default adds a few states per (segment, head) to the
    # records; the single pass holds those states only, bounded by the segment count
    big = (1, 131072, 32, 0, 64, 0)
    assert ws(*big) == path_ws(kda.KDA_PATH_AUTO, *big)
    assert record_ws(*big) < ws(*big) < record_ws(*big) + single_ws(*big) + 4096
    assert single_ws(*big) < 64 * 2**20 < record_ws(*big)
    assert single_ws(*big) <= single_ws(1, 8192, 32, 0, 64, 0) * 1.5
    # the automatic choice: the segment-parallel kernels from 4096 (chunk, head) pairs,
    # whatever the sequence length (the chunk bound of a packed batch counts)
    seg = lambda *a: path_ws(kda.KDA_PATH_RECORD_SEGMENTED, *a)  # noqa: E731
    for shape in ((1, 4096, 32, 0, 64, 0), (1, 8192, 16, 0, 64, 0), (1, 4096, 16, 0, 64, 0), (2, 4096, 16, 0, 64, 0)):
        assert ws(*shape) == record_ws(*shape) < seg(*shape)
    for shape in ((2, 4096, 32, 0, 64, 0), (8, 4096, 32, 0, 64, 0), (1024, 64, 32, 0, 64, 0), (1, 8192, 32, 0, 64, 0),
                  (1, 32768, 32, 4, 64, 0), (1, 4000, 32, 100, 64, 0)):
        assert ws(*shape) == seg(*shape) > record_ws(*shape)
    # a varlen query bounds every split of the same tokens
    for path in (kda.KDA_PATH_AUTO, kda.KDA_PATH_RECORD, kda.KDA_PATH_SINGLE_PASS, kda.KDA_PATH_RECORD_SEGMENTED):
        assert path_ws(path, 1, 32768, 32, 4, 64, 0) >= path_ws(path, 1, 32768, 32, 0, 64, 0)
    assert ws(1, 64, 1, 0, 32, 0) == 0
    assert ws(1, 64, 0, 0, 64, 0) == 0
    assert ws(1, 64, 1, 0, 64, 9) == 0
    bad = kda.Fusion()
    bad.prefill_path = 7
    assert L.kda_chunk_fwd_fused_workspace_size(1, 64, 1, 0, 64, 0, ctypes.byref(bad)) == 0


def fused_chunk_call(fusion, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, s0=None, cu=None, num_seqs=0, o=FAKE, fin=None,
                B=1, T=64, H=2, dk=128, dv=128, chunk=64, dtype=0)
    args.update(kw)
    a = args
    return L.kda_chunk_fwd_fused(a["q"], a["k"], a["v"], a["la"], a["beta"], a["s0"], a["cu"], a["num_seqs"],
                                 a["o"], a["fin"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["dtype"],
                                 None if fusion is None else ctypes.byref(fusion), None, 0, None)


def make_fusion(**kw):
    f = kda.Fusion(1, 1e-6, 1, 1, None, None, 1e-6)
    for k, v in kw.items():
        setattr(f, k, v)
    return f


@pytest.mark.parametrize("kw", [
    dict(qk_eps=-1.0),
    dict(norm_eps=float("nan")),
    dict(out_gate=1 << 20),                              # no norm weight
    dict(out_gate=(1 << 20) + 8, norm_weight=1 << 20),   # misaligned gate
    dict(out_gate=1 << 20, norm_weight=(1 << 20) + 4),   # misaligned weight
])
def test_fused_entry_points_reject_bad_fusion(kw):
    f = make_fusion(**kw)
    assert fused_chunk_call(f) == kda.KDA_ERR_INVALID_ARG
    assert L.kda_decode_step_fused(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 128, 128, 0,
                                   ctypes.byref(f), None) == kda.KDA_ERR_INVALID_ARG


def test_fused_entry_points_keep_the_plain_checks():
    f = make_fusion()
    assert fused_chunk_call(f, dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert fused_chunk_call(f, q=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert fused_chunk_call(f, B=0, q=None, k=None, v=None, la=None, beta=None, o=None) == kda.KDA_OK
    assert fused_chunk_call(None, B=0, q=None) == kda.KDA_OK
    assert L.kda_decode_step_fused(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 2, 128, 128, 0,
                                   ctypes.byref(f), None) == kda.KDA_ERR_INVALID_ARG
    assert L.kda_decode_step_fused(None, None, None, None, None, None, None, 0, 2, 128, 128, 0,
                                   ctypes.byref(f), None) == kda.KDA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(dv=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=3), kda.KDA_ERR_UNSUPPORTED),
    (dict(rows=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG),
    (dict(gate=None), kda.KDA_ERR_INVALID_ARG),
    (dict(weight=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(gate=ctypes.c_void_p(1 << 22), out=ctypes.c_void_p(1 << 22)), kda.KDA_ERR_INVALID_ARG),
    (dict(rows=0, o=None, gate=None), kda.KDA_OK),
])
def test_output_norm_gate_rejects(kw, status):
    a = dict(o=FAKE, gate=ctypes.c_void_p(1 << 21), weight=FAKE, out=ctypes.c_void_p(1 << 23), rows=16, dv=128,
             eps=1e-6, dtype=0)
    a.update(kw)
    assert L.kda_output_norm_gate(a["o"], a["gate"], a["weight"], a["out"], a["rows"], a["dv"], a["eps"],
                                  a["dtype"], None) == status


@pytest.mark.parametrize("gate,la,status", [
    (3, FAKE, kda.KDA_ERR_INVALID_ARG),                                  # not a kda_gate
    (-1, FAKE, kda.KDA_ERR_INVALID_ARG),
    (kda.KDA_GATE_HEAD, ctypes.c_void_p((1 << 20) + 2), kda.KDA_ERR_INVALID_ARG),     # scalar gate: 4-byte aligned
    (kda.KDA_GATE_CHANNEL, ctypes.c_void_p((1 << 20) + 4), kda.KDA_ERR_INVALID_ARG),  # channel gate: 16-byte
    (kda.KDA_GATE_CHANNEL, None, kda.KDA_ERR_INVALID_ARG),               # only the no-decay kind may omit it
    (kda.KDA_GATE_HEAD, None, kda.KDA_ERR_INVALID_ARG),
])
def test_gate_kind_checks(gate, la, status):
    f = make_fusion(gate_kind=gate)
    assert fused_chunk_call(f, la=la) == status
    assert L.kda_decode_step_fused(FAKE, FAKE, FAKE, la, FAKE, FAKE, FAKE, 4, 2, 128, 128, 0,
                                   ctypes.byref(f), None) == status


def bwd_call(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, s0=None, cu=None, num_seqs=0, do=FAKE, dfin=None,
             dq=FAKE, dk_=FAKE, dv_=FAKE, dla=FAKE, db=FAKE, ds0=None, B=1, T=64, H=2, dk=128, dv=128, dtype=0,
             ws=None, ws_bytes=0):
    return L.kda_chunk_bwd(q, k, v, la, beta, s0, cu, num_seqs, do, dfin, dq, dk_, dv_, dla, db, ds0, B, T, H, dk, dv,
                           dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=5), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(do=None), kda.KDA_ERR_INVALID_ARG),
    (dict(dq=None), kda.KDA_ERR_INVALID_ARG),
    (dict(dla=None), kda.KDA_ERR_INVALID_ARG),
    (dict(db=None), kda.KDA_ERR_INVALID_ARG),
    (dict(la=None), kda.KDA_ERR_INVALID_ARG),
    (dict(do=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(dla=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(ds0=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(dfin=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(db=ctypes.c_void_p((1 << 20) + 2)), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=2, B=2), kda.KDA_ERR_INVALID_ARG),
    (dict(ws=FAKE, ws_bytes=16), kda.KDA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=1 << 40), kda.KDA_ERR_INVALID_ARG),
])
def test_chunk_bwd_rejects(kw, status):
    assert bwd_call(**kw) == status
    assert L.kda_last_error()


def test_chunk_bwd_empty_batch_is_ok_without_device():
    assert bwd_call(B=0, T=0) == kda.KDA_OK
    assert bwd_call(cu=FAKE, num_seqs=0, T=0) == kda.KDA_OK


def test_bwd_workspace_size():
    # two 128 x 128 bf16 matrices per (16-token chunk, head) dominate
    n = kda.bwd_workspace_size(1, 4096, 16)
    assert n >= 4096 // 16 * 16 * 2 * 128 * 128 * 2
    assert kda.bwd_workspace_size(1, 4096, 16, dtype=kda.KDA_FP32) > n
    assert kda.bwd_workspace_size(1, 4096, 16, num_seqs=3) >= n
    assert kda.bwd_workspace_size(1, 64, 0) == 0


def dplr_call(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, la=FAKE, s0=None, cu=None, num_seqs=0, o=FAKE, fin=None,
              B=1, T=64, H=2, dk=128, dv=128, chunk=64, dtype=0, ws=None, ws_bytes=0):
    return L.kda_dplr_chunk_fwd(q, k, v, a, b, la, s0, cu, num_seqs, o, fin, B, T, H, dk, dv, chunk, dtype, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=16), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=5), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(a=None), kda.KDA_ERR_INVALID_ARG),
    (dict(b=None), kda.KDA_ERR_INVALID_ARG),
    (dict(la=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(a=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(b=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(fin=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=2, B=2), kda.KDA_ERR_INVALID_ARG),
    (dict(ws=FAKE, ws_bytes=16), kda.KDA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=1 << 40), kda.KDA_ERR_INVALID_ARG),
])
def test_dplr_rejects(kw, status):
    assert dplr_call(**kw) == status
    assert L.kda_last_error()


def test_dplr_empty_batch_is_ok_without_device():
    assert dplr_call(B=0, T=0) == kda.KDA_OK
    assert dplr_call(cu=FAKE, num_seqs=0, T=0) == kda.KDA_OK


def test_dplr_workspace_size():
    # one record of about 120 KiB (bf16) per (64-token chunk, head) dominates
    n = kda.dplr_workspace_size(1, 4096, 16)
    assert n >= 4096 // 64 * 16 * 120 * 1024
    assert kda.dplr_workspace_size(1, 4096, 16, dtype=kda.KDA_FP32) > n
    assert kda.dplr_workspace_size(1, 4096, 16, num_seqs=3) >= n
    assert kda.dplr_workspace_size(1, 64, 0) == 0
    assert kda.dplr_workspace_size(1, 64, 2) > kda.workspace_size(1, 64, 2, path="record")


def noalloc_call(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, s0=None, cu=None, num_seqs=0, o=FAKE, fin=FAKE,
                 B=1, T=64, H=2, dk=128, dv=128, chunk=64, dtype=0):
    return L.kda_chunk_fwd_noalloc(q, k, v, la, beta, s0, cu, num_seqs, o, fin, B, T, H, dk, dv, chunk, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=64), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(la=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=MISALIGNED), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=FAKE, num_seqs=2, B=2), kda.KDA_ERR_INVALID_ARG),
    # more scratch than the static array holds: 64 sequences x 64 heads (single pass),
    # and fp32 16-token chunks over 65536 tokens x 32 heads (records)
    (dict(B=64, T=8192, H=64), kda.KDA_ERR_WORKSPACE),
    (dict(dtype=1, chunk=16, T=65536, H=32), kda.KDA_ERR_WORKSPACE),
])
def test_chunk_fwd_noalloc_rejects(kw, status):
    """Every check, the scratch limit included, runs before any HIP call."""
    assert noalloc_call(**kw) == status
    assert L.kda_last_error().decode() != ""


def test_chunk_fwd_noalloc_limit():
    """The static scratch (KDA_NOALLOC_SCRATCH_BYTES) holds the single pass of the
    131072-token x 32-head workload; the rejected cases above need more."""
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == kda.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert kda.workspace_size(1, 131072, 32, path="single") <= limit
    assert kda.workspace_size(64, 8192, 64, path="single") > limit
    assert kda.workspace_size(1, 65536, 32, chunk=16, dtype=kda.KDA_FP32) > limit
    assert noalloc_call(B=0, q=None, k=None, v=None, la=None, beta=None, o=None, fin=None) == kda.KDA_OK
