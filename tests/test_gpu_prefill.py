"""Parity of the chunked prefill (kda_chunk_fwd, through the C ABI) with the fp64
oracle on MI355X. Small cases are compared element by element on every output;
the full-size workloads are compared on sampled heads and value columns, which the
oracle computes exactly (columns of the state evolve independently)."""
import numpy as np
import pytest
import torch

from parity import TOL, compare_prefill, gpu_prefill, normwise, oracle_prefill, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs  # noqa: E402


def small(seed, T, H, dtype, chunk, B=1, s0=0.3, la_scale=0.5, la_mode="scaled", cu=None):
    return inputs.make_prefill(seed, B=B, T=T, H=H, dtype=dtype, chunk=chunk, la_mode=la_mode, la_scale=la_scale,
                               s0_std=s0, cu_seqlens=cu)


def test_workload0_fp32_chunk16():
    """T=64, H=1, fp32, chunk 16, zero initial state: the fp32 gate (1e-4)."""
    compare_prefill(inputs.make_workload(0), label="workload0")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_ragged_multi_tile(dtype, chunk):
    """Several chunks, two sequences, a ragged last chunk, random initial state."""
    compare_prefill(small(11, T=200, H=3, dtype=dtype, chunk=chunk, B=2), label=f"ragged-{dtype}-c{chunk}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_varlen_edge_lengths(dtype):
    """Packed sequences of length 0, 1, 15, 16, 17, 63, 64, 65 and 130."""
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    compare_prefill(small(12, T=int(cu[-1]), H=2, dtype=dtype, chunk=64, cu=cu), label=f"varlen-{dtype}")


def test_null_initial_and_final_state():
    inp = small(13, T=100, H=2, dtype="bf16", chunk=64, s0=0.0)
    assert inp.initial_state is None
    o1, f1 = gpu_prefill(inp)
    from gated_delta_rule_57_amd import kda
    o2, f2 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, chunk=64, output_final_state=False)
    torch.cuda.synchronize()
    assert f2 is None
    assert torch.equal(o1, o2)
    z = torch.zeros_like(f1)
    o3, f3 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=z, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(f1, f3)


def test_in_place_final_state_and_workspace():
    inp = small(14, T=150, H=2, dtype="bf16", chunk=64)
    o1, f1 = gpu_prefill(inp)
    from gated_delta_rule_57_amd import kda
    st = inp.initial_state.clone()
    ws = torch.empty(kda.workspace_size(1, 150, 2, 0, 64, kda.KDA_BF16), dtype=torch.uint8, device="cuda")
    o2, f2 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=st, final_state=st,
                           chunk=64, workspace=ws)
    torch.cuda.synchronize()
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(f1, st)


def test_empty_sequences_copy_state():
    from gated_delta_rule_57_amd import kda
    s0 = torch.randn(3, 2, 128, 128, device="cuda")
    e = torch.zeros(3, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    la = torch.zeros(3, 0, 2, 128, device="cuda")
    b = torch.zeros(3, 0, 2, device="cuda")
    o, f = kda.chunk_fwd(e, e, e, la, b, initial_state=s0, chunk=64)
    torch.cuda.synchronize()
    assert o.shape == (3, 0, 2, 128) and torch.equal(f, s0)
    o, f = kda.chunk_fwd(e, e, e, la, b, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(f) == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_adversarial_decay_takes_fallback(dtype):
    """Per-token decays of -20 and -200 on some channels push a diagonal sub-block
    past the factoring range; the element-wise branch keeps the result exact."""
    inp = small(15, T=160, H=2, dtype=dtype, chunk=64, la_scale=0.05)
    la = inp.log_alpha
    la[:, 5, :, :32] = -20.0
    la[:, 40:46, 1, 32:64] = -200.0
    la[:, 100, 0, :] = -200.0
    la[:, 130:140, :, 100:] = -30.0
    compare_prefill(inp, label=f"adversarial-{dtype}")


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("case", ["fast12", "fast6", "two_sided"])
def test_fp32_fast_decay_runs(case, chunk):
    """fp32, every key channel: 12 tokens of -200 or 6 of -1000 next to slow rows of
    the same sub-chunk, and -200 rows at both ends of one sub-chunk. Every in-chunk
    exponent is a running sum of the decays it spans, so pairs of slow rows next to
    a fast run keep full fp32 accuracy: well inside the 1e-4 gate."""
    inp = small(19, T=192, H=2, dtype="fp32", chunk=chunk, la_scale=0.1)
    la = inp.log_alpha
    if case == "fast12":
        la[:, 20:32] = -200.0
        la[:, 130:142, 1] = -200.0
    elif case == "fast6":
        la[:, 0:6] = -1000.0
        la[:, 100:106, 0] = -1000.0
    else:
        la[:, 16] = -200.0
        la[:, 31] = -200.0
        la[:, 144, 1] = -200.0
        la[:, 159, 1] = -200.0
    eo, ef = compare_prefill(inp, label=f"fp32-{case}-c{chunk}")
    assert eo <= 1e-5 and ef <= 1e-5, (eo, ef)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chunk_size_does_not_change_result(dtype):
    inp = small(16, T=300, H=2, dtype=dtype, chunk=64)
    o64, f64 = gpu_prefill(inp, chunk=64)
    o16, f16 = gpu_prefill(inp, chunk=16)
    tol = TOL[dtype]
    assert normwise(o16.float().cpu().numpy(), o64.float().cpu().numpy()) <= tol
    assert normwise(f16.cpu().numpy(), f64.cpu().numpy()) <= tol


def test_beta_one_retrieval():
    """beta = 1, q = k, |k| = 1: the output of every token is its own value."""
    inp = small(17, T=256, H=2, dtype="fp32", chunk=64, la_scale=1.0)
    inp.beta.fill_(1.0)
    inp.q.copy_(inp.k)
    o, _ = gpu_prefill(inp)
    err = (o - inp.v).abs().max().item() / inp.v.abs().max().item()
    say(f"[retrieval] err={err:.3e}")
    assert err < 1e-4


def test_deterministic():
    inp = small(18, T=1000, H=4, dtype="bf16", chunk=64)
    o1, f1 = gpu_prefill(inp)
    o2, f2 = gpu_prefill(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_workload1_full():
    """T=4096, H=16, bf16, chunk 64, random initial state: every output compared."""
    compare_prefill(inputs.make_workload(1), label="workload1")


def compare_by_head_groups(inp, outs, group=8, label=""):
    """Compares full-size outputs with the oracle head group by head group (heads
    evolve independently), so host memory holds one group of fp64 outputs at a
    time. ``outs`` maps a label to a (o, final_state) pair of device tensors; the
    error is normwise over the whole tensor."""
    import oracle
    x = inp.numpy()
    s0 = None if x["initial_state"] is None else x["initial_state"].astype(np.float64)
    H = inp.q.shape[2]
    host = {k: (o.float().cpu().numpy(), fin.cpu().numpy()) for k, (o, fin) in outs.items()}
    acc = {k: [0.0, 0.0, 0.0, 0.0] for k in outs}  # max err o, max ref o, max err S, max ref S
    for h0 in range(0, H, group):
        hs = list(range(h0, min(H, h0 + group)))
        o_ref, f_ref = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], s0,
                                      cu_seqlens=x["cu_seqlens"], heads=hs)
        for k, (o_g, f_g) in host.items():
            a = acc[k]
            a[0] = max(a[0], float(np.max(np.abs(o_g[:, :, hs].astype(np.float64) - o_ref))))
            a[1] = max(a[1], float(np.max(np.abs(o_ref))))
            a[2] = max(a[2], float(np.max(np.abs(f_g[:, hs].astype(np.float64) - f_ref))))
            a[3] = max(a[3], float(np.max(np.abs(f_ref))))
        say(f"[parity] {label}: heads {hs[0]}..{hs[-1]} done")
    tol = TOL[inp.dtype]
    for k, a in acc.items():
        assert np.all(np.isfinite(host[k][0])) and np.all(np.isfinite(host[k][1]))
        eo, ef = a[0] / a[1], a[2] / a[3]
        say(f"[parity] {label} {k}: err_o={eo:.3e} err_state={ef:.3e} tol={tol:.0e}")
        assert eo <= tol and ef <= tol, (k, eo, ef)


@pytest.mark.timeout(600)
def test_workload2_varlen_all_heads():
    """4 packed sequences, 32768 tokens, H=32: every head and column compared, in the
    launch configuration the bench times and on the record path."""
    inp = inputs.make_workload(2)
    say(f"[parity] workload2 shape={tuple(inp.q.shape)} seqs={inp.num_seqs}")
    outs = {p: gpu_prefill(inp, path=p) for p in ("auto", "record")}
    compare_by_head_groups(inp, outs, label="workload2")


@pytest.mark.timeout(900)
def test_workload3_long_context_all_heads():
    """T=131072, H=32, bf16, mixed slow/fast decays: every head and column of o and
    the final state compared with the oracle over all 131072 tokens, for the
    automatic kernel choice the bench times and for each prefill path."""
    inp = inputs.make_workload(3)
    say(f"[parity] workload3 shape={tuple(inp.q.shape)}")
    outs = {p: gpu_prefill(inp, path=p) for p in ("auto", "record", "single")}
    compare_by_head_groups(inp, outs, label="workload3")
