"""Parity of every prefill kernel set for bf16 with 64-token chunks (kda_prefill_path:
the record path with slab state kernels, the record path with segment-parallel state
kernels, and the single pass) with the fp64 oracle on MI355X, through the C ABI.

The cases are small enough for the oracle to check every output, and chosen so that
the segment-parallel kernels cut each sequence into many one-chunk segments: the
first-segment output pass, the middle segments' (M, B) maps, the scan over them and
the later segments' output passes all run, over ragged and empty sequences."""
import numpy as np
import pytest
import torch

from oracle import fused as ofused
from parity import TOL, compare_prefill, normwise, oracle_prefill, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs, kda  # noqa: E402

PATHS = ["record", "segmented", "single"]


def run(inp, path, **kw):
    o, fin = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state,
                           cu_seqlens=inp.cu_seqlens, chunk=64, path=path, **kw)
    torch.cuda.synchronize()
    return o, fin


def check(inp, path, label):
    say(f"[paths] {label} path={path} shape={tuple(inp.q.shape)} seqs={inp.num_seqs}")
    o, fin = run(inp, path)
    o_ref, f_ref = oracle_prefill(inp)
    eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
    say(f"[paths] {label} path={path}: err_o={eo:.3e} err_state={ef:.3e}")
    assert np.isfinite(eo) and np.isfinite(ef)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    return o, fin


@pytest.mark.parametrize("path", PATHS)
def test_ragged_batch(path):
    """Two sequences of 200 tokens (four chunks, the last of 8 tokens), random initial state."""
    inp = inputs.make_prefill(51, B=2, T=200, H=3, dtype="bf16", la_scale=0.5, s0_std=0.3)
    check(inp, path, "ragged")


@pytest.mark.parametrize("path", PATHS)
def test_varlen_edge_lengths(path):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 0, 257]
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = inputs.make_prefill(52, B=1, T=int(cu[-1]), H=2, dtype="bf16", la_scale=0.5, s0_std=0.3,
                              cu_seqlens=cu)
    check(inp, path, "varlen")


@pytest.mark.parametrize("path", PATHS)
def test_long_scan(path):
    """41 chunks of one sequence and two heads: 41 one-chunk segments, a 39-step scan."""
    inp = inputs.make_prefill(53, B=1, T=64 * 40 + 37, H=2, dtype="bf16", la_scale=0.05, s0_std=0.3)
    check(inp, path, "long-scan")


@pytest.mark.parametrize("path", PATHS)
def test_adversarial_decay(path):
    """Decays of -20 and -200 on some channels: sub-chunks past the factoring range."""
    inp = inputs.make_prefill(54, B=1, T=300, H=2, dtype="bf16", la_scale=0.05, s0_std=0.3)
    la = inp.log_alpha
    la[:, 5, :, :32] = -20.0
    la[:, 40:46, 1, 32:64] = -200.0
    la[:, 100, 0, :] = -200.0
    la[:, 130:140, :, 100:] = -30.0
    check(inp, path, "adversarial")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("gate", ["head", "none"])
def test_scalar_gates(path, gate):
    inp = inputs.make_prefill(55, B=2, T=170, H=3, dtype="bf16", la_scale=0.5, s0_std=0.3, gate=gate)
    say(f"[paths] gate={gate} path={path}")
    o, fin = run(inp, path)
    x = inp.numpy()
    la = np.zeros(x["q"].shape, np.float32) if gate == "none" else \
        np.ascontiguousarray(np.broadcast_to(x["log_alpha"][..., None], x["q"].shape), dtype=np.float32)
    import oracle
    o_ref, f_ref = oracle.forward(x["q"], x["k"], x["v"], la, x["beta"], x["initial_state"].astype(np.float64))
    eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
    say(f"[paths] gate={gate} path={path}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("with_gate", [False, True])
def test_fused_prologue_epilogue(path, with_gate):
    """Raw q, k, gate and beta pre-activations, with and without the output RMSNorm and
    gate (fused into the segment-parallel kernels, a separate pass on the record path)."""
    r = inputs.make_raw_prefill(56, B=1, T=333, H=2, dtype="bf16", num_seqs=3, s0_std=0.2)
    f = kda.fusion(qk_eps=1e-6, out_gate=r.out_gate if with_gate else None,
                   norm_weight=r.norm_weight if with_gate else None, norm_eps=1e-5, path=path)
    o, fin = kda.chunk_fwd(r.q, r.k, r.v, r.gate, r.beta, initial_state=r.initial_state, cu_seqlens=r.cu_seqlens,
                           chunk=64, fusion=f)
    torch.cuda.synchronize()
    x = r.numpy()
    o_ref, f_ref = ofused.forward(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["initial_state"].astype(np.float64),
                                  x["cu_seqlens"], out_gate=x["out_gate"] if with_gate else None,
                                  norm_weight=x["norm_weight"], qk_eps=1e-6, norm_eps=1e-5)
    eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
    say(f"[paths] fused gate={with_gate} path={path}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("path", PATHS)
def test_state_aliasing_and_nulls(path):
    """final_state may be initial_state; a null initial state is zeros; a null final
    state is not written; the outputs do not change between these calls."""
    inp = inputs.make_prefill(57, B=2, T=260, H=2, dtype="bf16", la_scale=0.5, s0_std=0.3)
    o1, f1 = run(inp, path)
    st = inp.initial_state.clone()
    o2, f2 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=st, final_state=st, chunk=64,
                           path=path)
    o3, f3 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state,
                           chunk=64, path=path, output_final_state=False)
    z = torch.zeros_like(st)
    o4, f4 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, chunk=64, path=path)
    o5, f5 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=z, chunk=64, path=path)
    torch.cuda.synchronize()
    assert f2.data_ptr() == st.data_ptr() and f3 is None
    assert torch.equal(o1, o2) and torch.equal(f1, st) and torch.equal(o1, o3)
    assert torch.equal(o4, o5) and torch.equal(f4, f5)


@pytest.mark.parametrize("path", PATHS)
def test_empty_sequences_copy_state(path):
    s0 = torch.randn(3, 2, 128, 128, device="cuda")
    e = torch.zeros(3, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    la = torch.zeros(3, 0, 2, 128, device="cuda")
    b = torch.zeros(3, 0, 2, device="cuda")
    o, f = kda.chunk_fwd(e, e, e, la, b, initial_state=s0, chunk=64, path=path)
    torch.cuda.synchronize()
    assert o.shape == (3, 0, 2, 128) and torch.equal(f, s0)


@pytest.mark.parametrize("path", PATHS)
def test_explicit_workspace_and_determinism(path):
    """A caller workspace of exactly the queried size; two runs are bitwise equal."""
    inp = inputs.make_prefill(58, B=1, T=1000, H=4, dtype="bf16", la_scale=0.3, s0_std=0.1)
    n = kda.workspace_size(1, 1000, 4, 0, 64, kda.KDA_BF16, path=path)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o1, f1 = run(inp, path, workspace=ws)
    o2, f2 = run(inp, path, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    with pytest.raises(kda.KdaError):
        run(inp, path, workspace=ws[: n - 256])


def test_paths_agree_at_4k():
    """The 4K x 16-head workload on every path, each against the oracle on all outputs."""
    inp = inputs.make_workload(1)
    for path in PATHS:
        compare_prefill(inp, label=f"workload1-{path}", path=path)


def _many_lengths(seed, n, hi):
    """n sequence lengths drawn uniformly from [0, hi], about one in ten of them zero."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi + 1, size=n)
    lens[rng.random(n) < 0.1] = 0
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("path", PATHS)
def test_many_sequences(path):
    """1,500 packed sequences of 0 to 150 tokens (more than one 1,024-sequence block of
    the chunk and segment plans), random initial states."""
    cu = _many_lengths(61, 1500, 150)
    inp = inputs.make_prefill(61, B=1, T=int(cu[-1]), H=2, dtype="bf16", la_scale=0.3, s0_std=0.2,
                              cu_seqlens=cu)
    check(inp, path, "many-seqs")


@pytest.mark.parametrize("dtype,chunk", [("fp32", 16), ("fp32", 64), ("bf16", 16)])
def test_many_sequences_other_kernels(dtype, chunk):
    """The same packing on the fp32 and 16-token kernels."""
    cu = _many_lengths(62, 1300, 100)
    inp = inputs.make_prefill(62, B=1, T=int(cu[-1]), H=2, dtype=dtype, chunk=chunk, la_scale=0.3, s0_std=0.2,
                              cu_seqlens=cu)
    compare_prefill(inp, label=f"many-seqs {dtype} C={chunk}")


@pytest.mark.parametrize("path", PATHS + ["auto"])
def test_workspace_shared_by_uniform_and_packed_calls(path):
    """One workspace for a batch of equal sequences (whose chunk table the intra-chunk
    kernel writes) and then a packed batch (whose table the plan kernel writes), and
    back: every call matches the oracle."""
    uni = inputs.make_prefill(71, B=3, T=300, H=2, dtype="bf16", la_scale=0.3, s0_std=0.2)
    cu = np.array([0, 70, 70, 300, 641], dtype=np.int64)
    pk = inputs.make_prefill(72, B=1, T=641, H=2, dtype="bf16", la_scale=0.3, s0_std=0.2, cu_seqlens=cu)
    n = max(kda.workspace_size(3, 300, 2, 0, 64, kda.KDA_BF16, path=path),
            kda.workspace_size(1, 641, 2, 4, 64, kda.KDA_BF16, path=path))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for inp, label in ((uni, "uniform"), (pk, "packed"), (uni, "uniform again")):
        say(f"[paths] shared workspace {label} path={path}")
        o, fin = run(inp, path, workspace=ws)
        o_ref, f_ref = oracle_prefill(inp)
        eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
        say(f"[paths] shared workspace {label} path={path}: err_o={eo:.3e} err_state={ef:.3e}")
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
