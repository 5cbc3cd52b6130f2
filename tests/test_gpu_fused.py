"""Parity of the fused layer core (kda_chunk_fwd_fused, kda_decode_step_fused and
kda_output_norm_gate, through the C ABI) with the fp64 oracle's prologue and
epilogue (oracle/fused.py) on MI355X: raw q and k, gate and beta pre-activations,
and the output RMSNorm times a sigmoid gate."""
import numpy as np
import pytest
import torch

from oracle import fused as ofused
from parity import TOL, normwise, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs, kda  # noqa: E402

QK_EPS, NORM_EPS = 1e-6, 1e-5


def run_fused(r, with_gate, heads=None, chunk=None):
    f = kda.fusion(qk_eps=QK_EPS, out_gate=r.out_gate if with_gate else None,
                   norm_weight=r.norm_weight if with_gate else None, norm_eps=NORM_EPS)
    o, fin = kda.chunk_fwd(r.q, r.k, r.v, r.gate, r.beta, initial_state=r.initial_state, cu_seqlens=r.cu_seqlens,
                           chunk=chunk or r.chunk, fusion=f)
    torch.cuda.synchronize()
    x = r.numpy()
    s0 = None if x["initial_state"] is None else x["initial_state"].astype(np.float64)
    o_ref, fin_ref = ofused.forward(x["q"], x["k"], x["v"], x["gate"], x["beta"], s0, x["cu_seqlens"],
                                    out_gate=x["out_gate"] if with_gate else None, norm_weight=x["norm_weight"],
                                    qk_eps=QK_EPS, norm_eps=NORM_EPS, heads=heads)
    hs = slice(None) if heads is None else list(heads)
    eo = normwise(o.float().cpu().numpy()[:, :, hs], o_ref)
    ef = normwise(fin.cpu().numpy()[:, hs], fin_ref)
    return eo, ef


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_gate", [False, True])
@pytest.mark.parametrize("chunk", [16, 64])
def test_fused_prefill_small(dtype, with_gate, chunk):
    r = inputs.make_raw_prefill(21, B=2, T=150, H=3, dtype=dtype, chunk=chunk, s0_std=0.2)
    say(f"[fused] prefill {dtype} gate={with_gate} chunk={chunk}")
    eo, ef = run_fused(r, with_gate)
    say(f"[fused] prefill {dtype} gate={with_gate} chunk={chunk}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_prefill_varlen(dtype):
    r = inputs.make_raw_prefill(22, B=1, T=517, H=2, dtype=dtype, num_seqs=5)
    say(f"[fused] varlen {dtype} cu={r.cu_seqlens.tolist()}")
    eo, ef = run_fused(r, True)
    say(f"[fused] varlen {dtype}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_fused_prefill_4k_sampled_heads():
    """The 4K x 16-head prefill shape with raw inputs, compared on sampled heads."""
    r = inputs.make_raw_prefill(23, B=1, T=4096, H=16, dtype="bf16", s0_std=0.02)
    say("[fused] 4K x 16 heads, heads 0, 7, 15")
    eo, ef = run_fused(r, True, heads=[0, 7, 15])
    say(f"[fused] 4K: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_fusion_off_fields_match_plain_call():
    """A kda_fusion with every field off is the plain recurrence, bit for bit."""
    inp = inputs.make_prefill(24, B=1, T=200, H=2, dtype="bf16", la_scale=0.5, s0_std=0.1)
    o1, f1 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state)
    off = kda.fusion(normalize_qk=False, gate_preactivation=False, beta_preactivation=False)
    o2, f2 = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state, fusion=off)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("with_gate", [False, True])
def test_fused_decode_steps(dtype, with_gate):
    g = torch.Generator(device="cuda").manual_seed(25)
    N, H, steps = 5, 3, 6
    td = inputs.TORCH_DTYPE[dtype]
    rn = lambda *s: torch.randn(s, generator=g, device="cuda")  # noqa: E731
    state = 0.3 * rn(N, H, 128, 128)
    ref_state = state.double().cpu().numpy().copy()
    w = 0.5 + torch.rand(128, generator=g, device="cuda")
    say(f"[fused] decode {dtype} gate={with_gate}")
    worst = 0.0
    for _ in range(steps):
        q, k, v = (3.0 * rn(N, H, 128)).to(td), (3.0 * rn(N, H, 128)).to(td), rn(N, H, 128).to(td)
        a, b, z = rn(N, H, 128) - 3.0, rn(N, H), rn(N, H, 128).to(td)
        f = kda.fusion(qk_eps=QK_EPS, out_gate=z if with_gate else None, norm_weight=w if with_gate else None,
                       norm_eps=NORM_EPS)
        o = kda.decode_step(q, k, v, a, b, state, fusion=f)
        c = lambda t: t.float().cpu().numpy()  # noqa: E731
        o_ref = ofused.decode_step(c(q), c(k), c(v), c(a), c(b), ref_state, out_gate=c(z) if with_gate else None,
                                   norm_weight=c(w), qk_eps=QK_EPS, norm_eps=NORM_EPS)
        worst = max(worst, normwise(c(o), o_ref))
    es = normwise(state.cpu().numpy(), ref_state)
    say(f"[fused] decode {dtype} gate={with_gate}: err_o={worst:.3e} err_state={es:.3e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_output_norm_gate_standalone(dtype):
    g = torch.Generator(device="cuda").manual_seed(26)
    td = inputs.TORCH_DTYPE[dtype]
    rows = 1003  # not a multiple of the 8 rows of a work-group
    o = (5.0 * torch.randn((rows, 128), generator=g, device="cuda")).to(td)
    z = torch.randn((rows, 128), generator=g, device="cuda").to(td)
    w = 0.5 + torch.rand(128, generator=g, device="cuda")
    y = kda.output_norm_gate(o, z, w, eps=NORM_EPS)
    ref = ofused.output_norm_gate(o.float().cpu().numpy(), z.float().cpu().numpy(), w.cpu().numpy(), NORM_EPS)
    # bf16 output rounding is the only bf16 error here
    tol = 1e-5 if dtype == "fp32" else 8e-3
    err = normwise(y.float().cpu().numpy(), ref)
    say(f"[fused] outnorm {dtype}: err={err:.3e}")
    assert err <= tol
    o2 = o.clone()
    kda.output_norm_gate(o2, z, w, eps=NORM_EPS, out=o2)  # in place
    torch.cuda.synchronize()
    assert torch.equal(o2, y)


@pytest.mark.timeout(900)
def test_fused_full_size_sampled_heads():
    """T=131072, H=32, bf16: the bench's fused workload (raw q, k, gate and beta
    pre-activations, output RMSNorm and gate), all heads in one call; heads 3 and 30
    against the oracle's prologue, recurrence and epilogue run on those two heads."""
    r = inputs.make_raw_prefill(3, B=1, T=131072, H=32, dtype="bf16")
    f = kda.fusion(qk_eps=QK_EPS, out_gate=r.out_gate, norm_weight=r.norm_weight, norm_eps=NORM_EPS)
    say(f"[fused] full size shape={tuple(r.q.shape)}")
    o, fin = kda.chunk_fwd(r.q, r.k, r.v, r.gate, r.beta, initial_state=r.initial_state, chunk=64, fusion=f)
    torch.cuda.synchronize()
    heads = [3, 30]
    sl = lambda t: np.ascontiguousarray(t[:, :, heads].float().cpu().numpy())
    s0 = None if r.initial_state is None else r.initial_state[:, heads].cpu().numpy().astype(np.float64)
    o_ref, fin_ref = ofused.forward(sl(r.q), sl(r.k), sl(r.v), sl(r.gate), sl(r.beta), s0, None,
                                    out_gate=sl(r.out_gate), norm_weight=r.norm_weight.float().cpu().numpy(),
                                    qk_eps=QK_EPS, norm_eps=NORM_EPS)
    eo = normwise(sl(o), o_ref)
    ef = normwise(fin[:, heads].cpu().numpy(), fin_ref)
    say(f"[fused] full size: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
