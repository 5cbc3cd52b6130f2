"""Parity of the decode step (kda_decode_step, through the C ABI) with the fp64
oracle on MI355X, including the full 256-sequence x 32-head batch the bench times,
chained steps, and equivalence with prefill."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, normwise, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs, kda  # noqa: E402


def run_steps(dec, steps, sel=None):
    """Runs ``steps`` GPU decode steps and the oracle on the same inputs. ``sel`` =
    (sequence indices, head indices) restricts the oracle side. Returns the worst
    normwise errors on o and on the state."""
    state = dec.initial_state.clone()
    if sel is None:
        ref_state = dec.initial_state.double().cpu().numpy().copy()
    else:
        ns, hs = sel
        ref_state = np.ascontiguousarray(dec.initial_state[ns][:, hs].double().cpu().numpy())
    worst_o = 0.0
    for i in range(steps):
        o = kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], state)
        f = lambda t: t.float().cpu().numpy()
        xs = [dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i]]
        if sel is not None:
            xs = [x[ns][:, hs] for x in xs]
        o_ref = oracle.decode_step(*map(f, xs), ref_state)
        o_g = f(o) if sel is None else f(o[ns][:, hs])
        worst_o = max(worst_o, normwise(o_g, o_ref))
    torch.cuda.synchronize()
    s_g = state.cpu().numpy() if sel is None else state[ns][:, hs].cpu().numpy()
    return worst_o, normwise(s_g, ref_state)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_small_batch_many_steps(dtype):
    dec = inputs.make_decode(seed=40, N=3, H=2, n_steps=64, dtype=dtype, s0_std=0.3)
    say(f"[decode] small {dtype}")
    eo, es = run_steps(dec, 64)
    say(f"[decode] small {dtype}: err_o={eo:.3e} err_state={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_workload4_full_batch():
    """The measured batch: 256 sequences x 32 heads, every state and output compared
    over 8 consecutive steps."""
    dec = inputs.make_decode(n_steps=8)
    say("[decode] workload4 full batch, 8 steps")
    eo, es = run_steps(dec, 8)
    say(f"[decode] workload4: err_o={eo:.3e} err_state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.timeout(900)
def test_workload4_whole_chain():
    """The measured batch run as the workload defines it: 1024 successive steps of
    256 sequences x 32 heads. Every output of every step is compared with the fp64
    oracle chained over the same inputs, and every state after each of the first 8
    and the last 8 steps."""
    steps = 1024
    dec = inputs.make_decode(n_steps=steps)
    say(f"[decode] workload4 whole chain, {steps} steps")
    state = dec.initial_state.clone()
    ref_state = dec.initial_state.double().cpu().numpy()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    err_o = [0.0, 0.0]  # max |gpu - ref| and max |ref| over every output
    worst_s = 0.0
    for i in range(steps):
        o = kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], state)
        o_ref = oracle.decode_step(f(dec.q[i]), f(dec.k[i]), f(dec.v[i]), f(dec.log_alpha[i]), f(dec.beta[i]),
                                   ref_state)
        o_g = f(o).astype(np.float64)
        err_o[0] = max(err_o[0], float(np.max(np.abs(o_g - o_ref))))
        err_o[1] = max(err_o[1], float(np.max(np.abs(o_ref))))
        if i < 8 or i >= steps - 8:
            es = normwise(state.cpu().numpy(), ref_state)
            worst_s = max(worst_s, es)
            say(f"[decode] step {i}: err_state={es:.3e}")
        elif i % 128 == 0:
            say(f"[decode] step {i}: err_o so far={err_o[0] / err_o[1]:.3e}")
    eo = err_o[0] / err_o[1]
    say(f"[decode] workload4 whole chain: err_o={eo:.3e} err_state={worst_s:.3e}")
    assert np.isfinite(eo) and eo <= TOL["bf16"] and worst_s <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_steps_match_prefill(dtype):
    """T decode steps and one T-token prefill compute the same thing."""
    T, H = 48, 2
    inp = inputs.make_prefill(41, B=2, T=T, H=H, dtype=dtype, chunk=16, la_scale=0.5, s0_std=0.2)
    o_p, f_p = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, initial_state=inp.initial_state, chunk=16)
    state = inp.initial_state.clone()
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(inp.q[:, t].contiguous(), inp.k[:, t].contiguous(), inp.v[:, t].contiguous(),
                                    inp.log_alpha[:, t].contiguous(), inp.beta[:, t].contiguous(), state))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    tol = TOL[dtype]
    assert normwise(o_d.float().cpu().numpy(), o_p.float().cpu().numpy()) <= tol
    assert normwise(state.cpu().numpy(), f_p.cpu().numpy()) <= tol


def test_resume_from_host_copy_is_bitwise():
    """Stopping after k steps, copying the state to the host and back, and going on
    gives bitwise the same result as an uninterrupted run."""
    dec = inputs.make_decode(seed=42, N=4, H=3, n_steps=12, s0_std=0.1)
    a = dec.initial_state.clone()
    for i in range(12):
        kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], a)
    b = dec.initial_state.clone()
    for i in range(5):
        kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], b)
    host = b.cpu()
    b = host.cuda()
    for i in range(5, 12):
        kda.decode_step(dec.q[i], dec.k[i], dec.v[i], dec.log_alpha[i], dec.beta[i], b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
