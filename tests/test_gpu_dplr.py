"""Parity of the general-DPLR chunked forward (kda_dplr_chunk_fwd, through the C ABI)
with the fp64 oracle on MI355X, on the same seeded inputs. Small cases compare every
output; the long-context case compares sampled heads and value columns, which the
oracle computes exactly because columns of the state evolve independently."""
import numpy as np
import pytest
import torch

import oracle
from parity import TOL, normwise, say

pytestmark = pytest.mark.gpu

from gated_delta_rule_57_amd import inputs  # noqa: E402


def gpu_dplr(x, **kw):
    from gated_delta_rule_57_amd import kda
    o, fin = kda.dplr_chunk_fwd(x.q, x.k, x.v, x.a, x.b, x.log_alpha, initial_state=x.initial_state,
                                cu_seqlens=x.cu_seqlens, **kw)
    torch.cuda.synchronize()
    return o, fin


def compare_dplr(x, heads=None, cols=None, tol=None, label=""):
    say(f"[dplr] {label} dtype={x.dtype} shape={tuple(x.q.shape)} seqs={x.num_seqs} heads={heads} cols={cols} "
        f"lowrank={x.meta['lowrank']}")
    o, fin = gpu_dplr(x)
    n = x.numpy()
    s0 = None if n["initial_state"] is None else n["initial_state"].astype(np.float64)
    o_ref, f_ref = oracle.dplr_forward(n["q"], n["k"], n["v"], n["a"], n["b"], n["log_alpha"], s0,
                                       cu_seqlens=n["cu_seqlens"], heads=heads, cols=cols)
    hs = slice(None) if heads is None else list(heads)
    c0, c1 = (0, x.v.shape[-1]) if cols is None else cols
    o_g = o.float().cpu().numpy()[:, :, hs, c0:c1]
    f_g = fin.cpu().numpy()[:, hs, :, c0:c1]
    eo, ef = normwise(o_g, o_ref), normwise(f_g, f_ref)
    tol = tol if tol is not None else TOL[x.dtype]
    say(f"[dplr] {label}: err_o={eo:.3e} err_state={ef:.3e} tol={tol:.0e}")
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(f_g))
    assert eo <= tol, f"o error {eo} > {tol}"
    assert ef <= tol, f"final state error {ef} > {tol}"
    return eo, ef


def small(seed, T, H, dtype, B=1, s0=0.3, la_scale=0.5, lowrank="tied", cu=None, num_seqs=None):
    x = inputs.make_dplr(seed, B=B, T=T, H=H, dtype=dtype, la_scale=la_scale, s0_std=s0, lowrank=lowrank,
                         num_seqs=num_seqs)
    if cu is not None:
        x.cu_seqlens = torch.as_tensor(np.asarray(cu), dtype=torch.int32, device="cuda")
    return x


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("lowrank", ["tied", "free"])
def test_ragged_multi_tile(dtype, lowrank):
    """Several chunks, two sequences, a ragged last chunk, random initial state."""
    compare_dplr(small(21, T=200, H=3, dtype=dtype, B=2, lowrank=lowrank), label=f"ragged-{dtype}-{lowrank}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_varlen_edge_lengths(dtype):
    """Packed sequences of length 0, 1, 15, 16, 17, 63, 64, 65 and 130."""
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 130, 0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = small(22, T=int(cu[-1]), H=2, dtype=dtype, s0=0.0, lowrank="free")
    x.cu_seqlens = torch.as_tensor(cu, dtype=torch.int32, device="cuda")
    x.initial_state = 0.3 * torch.randn(len(lens), 2, 128, 128, device="cuda")
    compare_dplr(x, label=f"varlen-{dtype}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_adversarial_decay_takes_exact_path(dtype):
    """Per-token decays of -20 and -200 on some channels push a diagonal sub-block
    past the factoring range; the exact branch keeps the result within tolerance."""
    x = small(23, T=160, H=2, dtype=dtype, la_scale=0.05)
    la = x.log_alpha
    la[:, 5, :, :32] = -20.0
    la[:, 40:46, 1, 32:64] = -200.0
    la[:, 100, 0, :] = -200.0
    la[:, 130:140, :, 100:] = -30.0
    compare_dplr(x, label=f"adversarial-{dtype}")


def test_kda_case_matches_the_kda_kernel():
    """a = -beta k, b = alpha * k with key beta k is KDA: the DPLR kernel on those
    inputs agrees with the KDA kernel (fp32, both through the C ABI)."""
    from gated_delta_rule_57_amd import kda
    kd = inputs.make_prefill(24, B=1, T=300, H=2, dtype="fp32", chunk=64, la_scale=0.3, s0_std=0.2)
    bk = kd.beta[..., None] * kd.k
    o_d, f_d = kda.dplr_chunk_fwd(kd.q, bk.contiguous(), kd.v, (-bk).contiguous(),
                                  (torch.exp(kd.log_alpha) * kd.k).contiguous(), kd.log_alpha,
                                  initial_state=kd.initial_state)
    o_k, f_k = kda.chunk_fwd(kd.q, kd.k, kd.v, kd.log_alpha, kd.beta, initial_state=kd.initial_state, chunk=64)
    torch.cuda.synchronize()
    eo = normwise(o_d.cpu().numpy(), o_k.cpu().numpy())
    ef = normwise(f_d.cpu().numpy(), f_k.cpu().numpy())
    say(f"[dplr] kda case: o {eo:.3e} state {ef:.3e}")
    assert eo <= 1e-4 and ef <= 1e-4


def test_null_initial_and_final_state_and_workspace():
    from gated_delta_rule_57_amd import kda
    x = small(25, T=150, H=2, dtype="bf16", s0=0.0)
    o1, f1 = gpu_dplr(x)
    o2, f2 = gpu_dplr(x, output_final_state=False)
    assert f2 is None and torch.equal(o1, o2)
    st = 0.1 * torch.randn_like(f1)
    ref_o, ref_f = kda.dplr_chunk_fwd(x.q, x.k, x.v, x.a, x.b, x.log_alpha, initial_state=st.clone())
    ws = torch.empty(kda.dplr_workspace_size(1, 150, 2, 0, kda.KDA_BF16), dtype=torch.uint8, device="cuda")
    o3, f3 = kda.dplr_chunk_fwd(x.q, x.k, x.v, x.a, x.b, x.log_alpha, initial_state=st, final_state=st, workspace=ws)
    torch.cuda.synchronize()
    assert f3.data_ptr() == st.data_ptr()
    assert torch.equal(o3, ref_o) and torch.equal(st, ref_f)


def test_empty_sequences_copy_state():
    from gated_delta_rule_57_amd import kda
    s0 = torch.randn(3, 2, 128, 128, device="cuda")
    e = torch.zeros(3, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    la = torch.zeros(3, 0, 2, 128, device="cuda")
    o, f = kda.dplr_chunk_fwd(e, e, e, e, e, la, initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (3, 0, 2, 128) and torch.equal(f, s0)


def test_deterministic():
    x = small(26, T=1000, H=4, dtype="bf16")
    o1, f1 = gpu_dplr(x)
    o2, f2 = gpu_dplr(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_4k_full():
    """T=4096, H=16, bf16, random initial state, the stable recipe: every output."""
    compare_dplr(inputs.make_dplr(1, B=1, T=4096, H=16, dtype="bf16", la_scale=0.1, s0_std=0.02), label="4k")


@pytest.mark.timeout(900)
def test_long_context_sampled():
    """T=131072, H=32, bf16, mixed slow/fast decays and the stable recipe, in the
    launch configuration the bench times: two heads, 32 value columns each, against
    the oracle over all 131072 tokens."""
    x = inputs.make_dplr(3, B=1, T=131072, H=32, dtype="bf16", la_mode="mixed")
    compare_dplr(x, heads=[3, 30], cols=(48, 80), label="long")
