"""Parity of the scalar-gate (Gated DeltaNet: one decay per token and head) and
no-decay (DeltaNet) paths of the library with the fp64 oracle on MI355X. The oracle
runs the same recurrence with the scalar decay broadcast over the key channels
(or zero), which its own pins tie to textbook Gated DeltaNet and DeltaNet."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fused as ofused
from parity import TOL, normwise, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs, kda  # noqa: E402


def channel_log_alpha(x, la):
    """The per-channel log decay the oracle takes: the scalar broadcast, or zeros."""
    if la is None:
        return np.zeros(x["q"].shape, np.float32)
    return np.ascontiguousarray(np.broadcast_to(la[..., None], x["q"].shape), dtype=np.float32)


def compare(inp, label, heads=None, chunk=None):
    say(f"[gates] {label} gate={inp.meta['gate']} dtype={inp.dtype} shape={tuple(inp.q.shape)} seqs={inp.num_seqs}")
    o, fin = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state,
                           cu_seqlens=inp.cu_seqlens, chunk=chunk or inp.chunk)
    torch.cuda.synchronize()
    x = inp.numpy()
    la = None if inp.log_alpha is None else x["log_alpha"]
    s0 = None if x["initial_state"] is None else x["initial_state"].astype(np.float64)
    o_ref, f_ref = oracle.forward(x["q"], x["k"], x["v"], channel_log_alpha(x, la), x["beta"], s0,
                                  cu_seqlens=x["cu_seqlens"], heads=heads)
    hs = slice(None) if heads is None else list(heads)
    eo = normwise(o.float().cpu().numpy()[:, :, hs], o_ref)
    ef = normwise(fin.cpu().numpy()[:, hs], f_ref)
    say(f"[gates] {label}: err_o={eo:.3e} err_state={ef:.3e}")
    assert np.isfinite(eo) and np.isfinite(ef)
    assert eo <= TOL[inp.dtype] and ef <= TOL[inp.dtype]


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_small_ragged(gate, dtype, chunk):
    inp = inputs.make_prefill(31, B=2, T=150, H=3, dtype=dtype, chunk=chunk, la_scale=0.5, s0_std=0.3, gate=gate)
    compare(inp, f"small-c{chunk}")


@pytest.mark.parametrize("gate", ["head", "none"])
def test_varlen(gate):
    lens = [0, 1, 17, 64, 65, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = inputs.make_prefill(32, B=1, T=int(cu[-1]), H=2, dtype="bf16", la_scale=0.5, s0_std=0.2, cu_seqlens=cu,
                              gate=gate)
    compare(inp, "varlen")


@pytest.mark.parametrize("chunk", [16, 64])
def test_fp32_scalar_fast_decay_runs(chunk):
    """fp32 scalar gate: runs of -200 beside slow rows inside one chunk; the pair
    decay takes its exponent from whichever running sum subtracts the smaller
    total, so the fp32 result stays well inside its gate."""
    inp = inputs.make_prefill(33, B=1, T=192, H=2, dtype="fp32", la_scale=0.1, s0_std=0.3, gate="head")
    inp.log_alpha[:, 2:8] = -200.0
    inp.log_alpha[:, 90:93, 1] = -200.0
    inp.log_alpha[:, 150] = -200.0
    o, fin = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state, chunk=chunk)
    torch.cuda.synchronize()
    x = inp.numpy()
    o_ref, f_ref = oracle.forward(x["q"], x["k"], x["v"], channel_log_alpha(x, x["log_alpha"]), x["beta"],
                                  x["initial_state"].astype(np.float64))
    eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
    say(f"[gates] fp32 scalar fast runs c{chunk}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= 1e-5 and ef <= 1e-5


def test_strong_scalar_decay_stays_finite():
    """Decays of ~20 nats per token: the pair factor 2^(gh_r - gh_s) underflows to 0
    for distant rows, never overflows."""
    inp = inputs.make_prefill(33, B=1, T=200, H=2, dtype="fp32", la_scale=20.0, s0_std=0.3, gate="head")
    compare(inp, "strong")


def test_4k_sampled_heads():
    inp = inputs.make_prefill(34, B=1, T=4096, H=16, dtype="bf16", la_scale=0.1, s0_std=0.02, gate="head")
    compare(inp, "4K", heads=[0, 9, 15])


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_steps(gate, dtype):
    g = torch.Generator(device="cuda").manual_seed(35)
    N, H, steps = 6, 3, 5
    td = inputs.TORCH_DTYPE[dtype]
    rn = lambda *s: torch.randn(s, generator=g, device="cuda")  # noqa: E731
    unit = lambda x: x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)  # noqa: E731
    state = 0.3 * rn(N, H, 128, 128)
    ref = state.double().cpu().numpy().copy()
    worst = 0.0
    say(f"[gates] decode gate={gate} {dtype}")
    for _ in range(steps):
        q, k, v = unit(rn(N, H, 128)).to(td), unit(rn(N, H, 128)).to(td), rn(N, H, 128).to(td)
        la = None if gate == "none" else -0.5 * torch.nn.functional.softplus(rn(N, H))
        b = torch.sigmoid(rn(N, H))
        o = kda.decode_step(q, k, v, la, b, state)
        c = lambda t: t.float().cpu().numpy()  # noqa: E731
        lac = np.zeros((N, H, 128), np.float32) if la is None else np.repeat(c(la)[..., None], 128, axis=-1)
        o_ref = oracle.decode_step(c(q), c(k), c(v), lac, c(b), ref)
        worst = max(worst, normwise(c(o), o_ref))
    es = normwise(state.cpu().numpy(), ref)
    say(f"[gates] decode gate={gate} {dtype}: err_o={worst:.3e} err_state={es:.3e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_scalar_gate_with_prologue():
    """The scalar gate from its pre-activation, with raw q, k and the output gate."""
    r = inputs.make_raw_prefill(36, B=1, T=230, H=2, dtype="bf16", s0_std=0.2)
    a = r.gate[..., 0].contiguous()   # one pre-activation per (token, head)
    f = kda.fusion(out_gate=r.out_gate, norm_weight=r.norm_weight, norm_eps=1e-5)
    o, fin = kda.chunk_fwd(r.q, r.k, r.v, a, r.beta, initial_state=r.initial_state, fusion=f)
    torch.cuda.synchronize()
    x = r.numpy()
    ab = np.ascontiguousarray(np.broadcast_to(a.cpu().numpy()[..., None], x["q"].shape), dtype=np.float32)
    o_ref, f_ref = ofused.forward(x["q"], x["k"], x["v"], ab, x["beta"], x["initial_state"].astype(np.float64),
                                  out_gate=x["out_gate"], norm_weight=x["norm_weight"], norm_eps=1e-5)
    eo, ef = normwise(o.float().cpu().numpy(), o_ref), normwise(fin.cpu().numpy(), f_ref)
    say(f"[gates] scalar gate + prologue: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("gate", ["head", "none"])
def test_full_size_sampled_heads(gate):
    """T=131072, H=32, bf16, chunk 64: the prefill workload with the scalar gate the
    bench times (its per-channel decay's first channel, or none), all heads in one
    call; heads 3 and 30 against the oracle run on those two heads alone."""
    inp = inputs.make_workload(3)
    la = inp.log_alpha[..., 0].contiguous() if gate == "head" else None
    say(f"[gates] full size gate={gate} shape={tuple(inp.q.shape)}")
    o, fin = kda.chunk_fwd(inp.q, inp.k, inp.v, la, inp.beta, initial_state=inp.initial_state, chunk=64)
    torch.cuda.synchronize()
    heads = [3, 30]
    f = lambda t: np.ascontiguousarray(t[:, :, heads].float().cpu().numpy())
    q = f(inp.q)
    la_c = np.zeros(q.shape, np.float32) if la is None else \
        np.ascontiguousarray(np.broadcast_to(f(la)[..., None], q.shape), dtype=np.float32)
    s0 = None if inp.initial_state is None else inp.initial_state[:, heads].cpu().numpy().astype(np.float64)
    o_ref, f_ref = oracle.forward(q, f(inp.k), f(inp.v), la_c, f(inp.beta), s0)
    eo = normwise(f(o), o_ref)
    ef = normwise(fin[:, heads].cpu().numpy(), f_ref)
    say(f"[gates] full size {gate}: err_o={eo:.3e} err_state={ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
