"""kda_chunk_fwd_noalloc (the prefill whose scratch is a static per-device array)
against kda_chunk_fwd on MI355X, through the C ABI: two calls in a row, the second
on a smaller input, so the second reuses scratch the first left behind."""
import numpy as np
import pytest
import torch

from parity import TOL, normwise, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs, kda  # noqa: E402


def check(inp, label):
    """The no-alloc call against kda_chunk_fwd (its default kernels) within the
    dtype's tolerance, and bitwise against kda_chunk_fwd on the kernels the no-alloc
    call runs (the single pass for bf16 with 64-token chunks)."""
    say(f"[noalloc] {label} dtype={inp.dtype} shape={tuple(inp.q.shape)} chunk={inp.chunk} seqs={inp.num_seqs}")
    args = (inp.q, inp.k, inp.v, inp.log_alpha, inp.beta)
    kw = dict(initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens, chunk=inp.chunk)
    o_ref, f_ref = kda.chunk_fwd(*args, **kw)
    same_path = "single" if (inp.dtype == "bf16" and inp.chunk == 64) else "auto"
    o_same, f_same = kda.chunk_fwd(*args, path=same_path, **kw)
    o = torch.empty_like(o_ref)
    fin = torch.empty_like(f_ref)
    o.fill_(float("nan"))
    fin.fill_(float("nan"))
    r_o, r_f = kda.chunk_fwd_noalloc(*args, o=o, final_state=fin, **kw)
    torch.cuda.synchronize()
    assert r_o.data_ptr() == o.data_ptr() and r_f.data_ptr() == fin.data_ptr()
    eo = normwise(o.float().cpu().numpy(), o_ref.float().cpu().numpy())
    ef = normwise(fin.cpu().numpy(), f_ref.cpu().numpy())
    say(f"[noalloc] {label}: against kda_chunk_fwd err_o={eo:.3e} err_state={ef:.3e}")
    assert np.isfinite(eo) and np.isfinite(ef)
    assert eo <= TOL[inp.dtype] and ef <= TOL[inp.dtype]
    assert torch.equal(o, o_same) and torch.equal(fin, f_same)


def test_two_calls_bf16_second_smaller():
    check(inputs.make_prefill(61, B=1, T=3000, H=4, dtype="bf16", num_seqs=3, la_scale=0.3, s0_std=0.3), "bf16 first")
    check(inputs.make_prefill(62, B=2, T=300, H=2, dtype="bf16", la_scale=0.3, s0_std=0.3), "bf16 second")


def test_two_calls_fp32_chunk16_second_smaller():
    check(inputs.make_prefill(63, B=2, T=400, H=3, dtype="fp32", chunk=16, la_scale=0.3, s0_std=0.3), "fp32 first")
    check(inputs.make_prefill(64, B=1, T=37, H=1, dtype="fp32", chunk=16, la_scale=0.3, s0_std=0.3), "fp32 second")


def test_long_context_workload_fits():
    """131072 tokens x 32 heads: the single pass's scratch fits the static array."""
    check(inputs.make_workload(3), "workload3")
    check(inputs.make_prefill(65, B=1, T=640, H=2, dtype="bf16", la_scale=0.3, s0_std=0.3), "after workload3")


def test_oversize_is_rejected():
    """12 sequences x 32 heads need 151 MB of per-segment states: rejected before any
    launch, and the outputs are left as they were."""
    q = torch.zeros(12, 64, 32, 128, dtype=torch.bfloat16, device="cuda")
    la = torch.zeros(12, 64, 32, 128, dtype=torch.float32, device="cuda")
    b = torch.zeros(12, 64, 32, dtype=torch.float32, device="cuda")
    o = torch.full_like(q, 7.0)
    assert kda.workspace_size(12, 64, 32, path="single") > kda.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kda.KdaError):
        kda.chunk_fwd_noalloc(q, q, q, la, b, o=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
