"""Seeded synthetic inputs for the KDA token mixer.

This module only draws random numbers and shapes them; it holds none of the
recurrence's arithmetic. The tests of the GPU path, the oracle comparisons and
the bench all take their inputs from here.

The measured workloads (``make_prefill``, ``make_workload``, ``make_decode``) are
drawn on the host with NumPy's ``default_rng`` in float64, so they can be
reproduced on any machine: every draw takes the next child of
``SeedSequence(seed)`` in a fixed order, and each block of ``BLOCK`` elements of a
draw comes from its own child stream of that child (so the values do not depend on
how many threads fill the blocks). Prefill draw order: cut points (packed batches),
q, k, v, log-decay normals, slow-channel choice (mixed mode), beta normals, initial
state. Decode: the initial state, then per step q, k, v, log-decay normals, beta
normals.

Distributions (the plainest reading of the workloads the library is measured on):
  q, k      ~ N(0, 1), then L2-normalised per (token, head) in float64 (the model
              normalises q and k before the mixer; GeekNews "Kimi Linear" summary,
              section "Kimi Linear 모델 구성"), then rounded to the compute dtype
              (bf16: round to nearest even, by torch on the CPU)
  v         ~ N(0, 1), rounded to the compute dtype
  log_alpha = -scale * softplus(N(0, 1)) per channel, computed in float64 and
              stored as float32. In "mixed" mode a seeded half of each head's
              channels is -1e-3 (slow) and the rest -softplus(N(0, 1)) (fast), the
              same channels at every token
  beta      = sigmoid(N(0, 1)) per (token, head), float32
  S_0       ~ N(0, s0_std) float32, or None (zeros)

The raw layer inputs of the fused path (``make_raw_prefill``), the general-DPLR
inputs (``make_dplr``) and the backward's cotangents (``make_cotangents``) are drawn
the same way, each with the draw order its docstring states.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

D = 128

#: The measured workloads, by index: shapes and distributions.
WORKLOADS = {
    0: dict(name="kda_fwd_T64_H1_fp32_c16", B=1, T=64, H=1, dtype="fp32", chunk=16,
            la_mode="scaled", la_scale=0.1, s0_std=0.0),
    1: dict(name="kda_prefill_T4096_H16_bf16", B=1, T=4096, H=16, dtype="bf16", chunk=64,
            la_mode="scaled", la_scale=0.1, s0_std=0.02),
    2: dict(name="kda_varlen_4seq_T32768_H32_bf16", B=1, T=32768, H=32, dtype="bf16", chunk=64,
            la_mode="scaled", la_scale=0.05, s0_std=0.0, num_seqs=4),
    3: dict(name="kda_prefill_T131072_H32_bf16", B=1, T=131072, H=32, dtype="bf16", chunk=64,
            la_mode="mixed", la_scale=1.0, s0_std=0.0),
    4: dict(name="kda_decode_N256_H32_bf16", N=256, H=32, dtype="bf16", steps=1024,
            la_scale=0.1, s0_std=0.02),
}

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass
class PrefillInputs:
    q: torch.Tensor          # [B, T, H, dk] compute dtype
    k: torch.Tensor          # [B, T, H, dk] compute dtype
    v: torch.Tensor          # [B, T, H, dv] compute dtype
    log_alpha: torch.Tensor  # [B, T, H, dk] fp32
    beta: torch.Tensor       # [B, T, H] fp32
    initial_state: Optional[torch.Tensor]  # [N, H, dk, dv] fp32, or None (zeros)
    cu_seqlens: Optional[torch.Tensor]     # int32 [N+1], or None
    dtype: str
    chunk: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    def numpy(self):
        """float32 NumPy copies (exact for bf16 and fp32 values) and int64 cu_seqlens."""
        f = lambda t: None if t is None else t.detach().float().cpu().numpy()
        cu = None if self.cu_seqlens is None else self.cu_seqlens.cpu().numpy().astype(np.int64)
        return dict(q=f(self.q), k=f(self.k), v=f(self.v), log_alpha=f(self.log_alpha), beta=f(self.beta),
                    initial_state=f(self.initial_state), cu_seqlens=cu)


#: Elements per independent stream of a host draw (a multiple of the head size).
BLOCK = 1 << 22


def _host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class HostDraws:
    """Host draws of one input set: each call takes the next child of
    ``SeedSequence(seed)``; block b of a draw (``BLOCK`` elements) comes from
    ``default_rng`` on that child's b-th child."""

    def __init__(self, seed: int):
        self.root = np.random.SeedSequence(int(seed))

    def child(self):
        return self.root.spawn(1)[0]

    def fill(self, n: int, fn, ss=None) -> np.ndarray:
        """n float32 values, block by block: fn(rng, count) returns count float64 values."""
        ss = ss if ss is not None else self.child()
        nb = (n + BLOCK - 1) // BLOCK
        kids = ss.spawn(nb)
        out = np.empty(n, np.float32)

        def work(b):
            lo = b * BLOCK
            c = min(BLOCK, n - lo)
            out[lo:lo + c] = fn(np.random.default_rng(kids[b]), c)

        if nb > 1:
            with ThreadPoolExecutor(_host_threads()) as ex:
                list(ex.map(work, range(nb)))
        elif nb == 1:
            work(0)
        return out


def _h_normal(rng, c):
    return rng.standard_normal(c)


def _h_unit_rows(rng, c, d=D):
    x = rng.standard_normal(c).reshape(-1, d)
    return (x / np.sqrt(np.sum(x * x, axis=1, keepdims=True))).ravel()


def _h_softplus(x):
    return np.logaddexp(0.0, x)


def _h_sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _to_device(a32: np.ndarray, shape, dtype: str, device):
    """float32 host values -> the compute dtype (bf16 rounded to nearest even by torch
    on the CPU) on ``device``."""
    t = torch.from_numpy(a32).view(*shape)
    if dtype != "fp32":
        t = t.to(TORCH_DTYPE[dtype])
    return t.to(device)


def _host_composition(rng, total: int, parts: int) -> np.ndarray:
    """cu_seqlens of ``parts`` positive lengths summing to ``total``: distinct cut
    points drawn uniformly from [1, total-1] and sorted."""
    cuts = np.sort(rng.choice(total - 1, size=parts - 1, replace=False) + 1)
    return np.concatenate([[0], cuts, [total]]).astype(np.int32)


def make_prefill(seed: int, B: int, T: int, H: int, dtype: str, chunk: int = 64, la_mode: str = "scaled",
                 la_scale: float = 0.1, s0_std: float = 0.0, num_seqs: Optional[int] = None,
                 cu_seqlens=None, device="cuda", dk: int = D, dv: int = D, gate: str = "channel") -> PrefillInputs:
    """``gate``: "channel" (log_alpha [B, T, H, dk]), "head" (one decay per (token,
    head): log_alpha [B, T, H], drawn like one channel) or "none" (log_alpha None)."""
    dr = HostDraws(seed)
    cu = None
    if cu_seqlens is not None:
        assert B == 1
        cu = torch.as_tensor(np.asarray(cu_seqlens), dtype=torch.int32).to(device)
    elif num_seqs is not None:
        assert B == 1
        cu = torch.from_numpy(_host_composition(np.random.default_rng(dr.child()), T, num_seqs)).to(device)
    shape_k, shape_v = (B, T, H, dk), (B, T, H, dv)
    nk, nv = B * T * H * dk, B * T * H * dv
    q = _to_device(dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk)), shape_k, dtype, device)
    k = _to_device(dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk)), shape_k, dtype, device)
    v = _to_device(dr.fill(nv, _h_normal), shape_v, dtype, device)
    if gate == "none":
        log_alpha = None
    elif gate == "head":
        assert la_mode == "scaled"
        log_alpha = _to_device(dr.fill(B * T * H, lambda r, c: -la_scale * _h_softplus(r.standard_normal(c))),
                               (B, T, H), "fp32", device)
    elif la_mode == "scaled":
        log_alpha = _to_device(dr.fill(nk, lambda r, c: -la_scale * _h_softplus(r.standard_normal(c))), shape_k,
                               "fp32", device)
    elif la_mode == "mixed":
        la = dr.fill(nk, lambda r, c: -_h_softplus(r.standard_normal(c))).reshape(B * T, H, dk)
        rs = np.random.default_rng(dr.child())
        for h in range(H):
            slow = rs.permutation(dk)[: dk // 2]
            la[:, h, slow] = np.float32(-1e-3)
        log_alpha = _to_device(la.reshape(-1), shape_k, "fp32", device)
    else:
        raise ValueError(la_mode)
    beta = _to_device(dr.fill(B * T * H, lambda r, c: _h_sigmoid(r.standard_normal(c))), (B, T, H), "fp32", device)
    N = B if cu is None else cu.numel() - 1
    s0 = None
    if s0_std > 0:
        s0 = _to_device(dr.fill(N * H * dk * dv, lambda r, c: s0_std * r.standard_normal(c)), (N, H, dk, dv), "fp32",
                        device)
    return PrefillInputs(q.contiguous(), k.contiguous(), v.contiguous(),
                         None if log_alpha is None else log_alpha.contiguous(), beta.contiguous(),
                         s0, cu, dtype, chunk, dict(seed=seed, la_mode=la_mode, la_scale=la_scale, gate=gate))


def make_cotangents(seed: int, inp: PrefillInputs, final_std: float = 0.1, device="cuda"):
    """Cotangents for a backward call on ``inp``: grad_o ~ N(0, 1) rounded to the input
    dtype, shaped like o, and grad_final_state ~ N(0, final_std^2) fp32 [N, H, dk, dv]
    (None when final_std is 0). Host draws from ``SeedSequence(seed + 1000)``, in that
    order."""
    dr = HostDraws(seed + 1000)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    grad_o = _to_device(dr.fill(B * T * H * dv, _h_normal), (B, T, H, dv), inp.dtype, device).contiguous()
    n = inp.num_seqs * H * dk * dv
    gf = (_to_device(dr.fill(n, lambda r, c: final_std * r.standard_normal(c)), (inp.num_seqs, H, dk, dv), "fp32",
                     device) if final_std > 0 else None)
    return grad_o, gf


def make_workload(idx: int, device="cuda", **overrides) -> PrefillInputs:
    """Prefill workload ``idx`` (0-3), seed = idx; ``overrides`` may change sizes for
    quicker variants (their draws then differ from the full size)."""
    w = dict(WORKLOADS[idx])
    w.update(overrides)
    return make_prefill(seed=w.get("seed", idx), B=w["B"], T=w["T"], H=w["H"], dtype=w["dtype"], chunk=w["chunk"],
                        la_mode=w["la_mode"], la_scale=w["la_scale"], s0_std=w["s0_std"],
                        num_seqs=w.get("num_seqs"), device=device)


@dataclass
class DecodeInputs:
    initial_state: torch.Tensor  # [N, H, dk, dv] fp32
    q: torch.Tensor              # [steps, N, H, dk] compute dtype
    k: torch.Tensor              # [steps, N, H, dk]
    v: torch.Tensor              # [steps, N, H, dv]
    log_alpha: torch.Tensor      # [steps, N, H, dk] fp32
    beta: torch.Tensor           # [steps, N, H] fp32
    dtype: str


def make_decode(seed: int = 4, N: int = 256, H: int = 32, n_steps: int = 1024, dtype: str = "bf16",
                la_scale: float = 0.1, s0_std: float = 0.02, device="cuda", dk: int = D, dv: int = D) -> DecodeInputs:
    """Decode workload: persisted states, then ``n_steps`` fresh single tokens per
    (sequence, head). Step i's draws do not depend on ``n_steps``."""
    dr = HostDraws(seed)
    s0 = _to_device(dr.fill(N * H * dk * dv, lambda r, c: s0_std * r.standard_normal(c)), (N, H, dk, dv), "fp32",
                    device)
    kids = [[dr.child() for _ in range(5)] for _ in range(n_steps)]  # q, k, v, log-decay, beta per step
    nk, nv = N * H * dk, N * H * dv

    def step(i):
        kq, kk, kv, kl, kb = kids[i]
        # one block per draw (a step's draws are far below BLOCK)
        return (dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk), kq), dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk), kk),
                dr.fill(nv, _h_normal, kv), dr.fill(nk, lambda r, c: -la_scale * _h_softplus(r.standard_normal(c)), kl),
                dr.fill(N * H, lambda r, c: _h_sigmoid(r.standard_normal(c)), kb))

    with ThreadPoolExecutor(_host_threads()) as ex:
        steps = list(ex.map(step, range(n_steps)))
    st = lambda j, shape, dt: _to_device(np.concatenate([x[j] for x in steps]) if steps else np.zeros(0, np.float32),
                                         (n_steps,) + shape, dt, device)
    return DecodeInputs(s0, st(0, (N, H, dk), dtype), st(1, (N, H, dk), dtype), st(2, (N, H, dv), dtype),
                        st(3, (N, H, dk), "fp32"), st(4, (N, H), "fp32"), dtype)


@dataclass
class RawPrefillInputs:
    """Inputs of the fused layer core (kda_fusion): raw projections and pre-activations."""
    q: torch.Tensor            # [B, T, H, dk] compute dtype, not normalised
    k: torch.Tensor            # [B, T, H, dk] compute dtype, not normalised
    v: torch.Tensor            # [B, T, H, dv] compute dtype
    gate: torch.Tensor         # [B, T, H, dk] fp32 pre-activation of the decay (log alpha = -softplus)
    beta: torch.Tensor         # [B, T, H] fp32 pre-activation of beta (beta = sigmoid)
    out_gate: torch.Tensor     # [B, T, H, dv] compute dtype, pre-activation of the output gate
    norm_weight: torch.Tensor  # [dv] fp32 RMSNorm weight
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    dtype: str
    chunk: int

    @property
    def num_seqs(self):
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    def numpy(self):
        f = lambda t: None if t is None else t.detach().float().cpu().numpy()
        cu = None if self.cu_seqlens is None else self.cu_seqlens.cpu().numpy().astype(np.int64)
        return dict(q=f(self.q), k=f(self.k), v=f(self.v), gate=f(self.gate), beta=f(self.beta),
                    out_gate=f(self.out_gate), norm_weight=f(self.norm_weight),
                    initial_state=f(self.initial_state), cu_seqlens=cu)


def make_raw_prefill(seed: int, B: int, T: int, H: int, dtype: str, chunk: int = 64, gate_shift: float = -3.0,
                     qk_scale: float = 3.0, s0_std: float = 0.0, num_seqs: Optional[int] = None, device="cuda",
                     dk: int = D, dv: int = D) -> RawPrefillInputs:
    """Raw layer inputs: q, k ~ qk_scale * N(0, 1) (not normalised); v ~ N(0, 1);
    gate ~ N(gate_shift, 1) (gate_shift = -3 gives log alpha = -softplus(gate) near
    -0.05, the decay range of the standard workloads); beta, out_gate ~ N(0, 1);
    norm_weight ~ U(0.5, 1.5). Host draws in the order: cut points, q, k, v, gate,
    beta, out_gate, norm_weight, initial state."""
    dr = HostDraws(seed)
    cu = None
    if num_seqs is not None:
        assert B == 1
        cu = torch.from_numpy(_host_composition(np.random.default_rng(dr.child()), T, num_seqs)).to(device)
    shape_k, shape_v = (B, T, H, dk), (B, T, H, dv)
    nk, nv = B * T * H * dk, B * T * H * dv
    q = _to_device(dr.fill(nk, lambda r, c: qk_scale * r.standard_normal(c)), shape_k, dtype, device)
    k = _to_device(dr.fill(nk, lambda r, c: qk_scale * r.standard_normal(c)), shape_k, dtype, device)
    v = _to_device(dr.fill(nv, _h_normal), shape_v, dtype, device)
    gate = _to_device(dr.fill(nk, lambda r, c: r.standard_normal(c) + gate_shift), shape_k, "fp32", device)
    beta = _to_device(dr.fill(B * T * H, _h_normal), (B, T, H), "fp32", device)
    out_gate = _to_device(dr.fill(nv, _h_normal), shape_v, dtype, device)
    w = _to_device(dr.fill(dv, lambda r, c: 0.5 + r.random(c)), (dv,), "fp32", device)
    N = B if cu is None else cu.numel() - 1
    s0 = None
    if s0_std > 0:
        s0 = _to_device(dr.fill(N * H * dk * dv, lambda r, c: s0_std * r.standard_normal(c)), (N, H, dk, dv), "fp32",
                        device)
    return RawPrefillInputs(q.contiguous(), k.contiguous(), v.contiguous(), gate.contiguous(), beta.contiguous(),
                            out_gate.contiguous(), w.contiguous(), s0, cu, dtype, chunk)


@dataclass
class DplrInputs:
    """Inputs of the general diagonal-plus-low-rank recurrence
    S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T."""
    q: torch.Tensor          # [B, T, H, dk] compute dtype
    k: torch.Tensor          # [B, T, H, dk] compute dtype
    v: torch.Tensor          # [B, T, H, dv] compute dtype
    a: torch.Tensor          # [B, T, H, dk] compute dtype
    b: torch.Tensor          # [B, T, H, dk] compute dtype
    log_alpha: torch.Tensor  # [B, T, H, dk] fp32
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    dtype: str
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    def numpy(self):
        f = lambda t: None if t is None else t.detach().float().cpu().numpy()
        cu = None if self.cu_seqlens is None else self.cu_seqlens.cpu().numpy().astype(np.int64)
        return dict(q=f(self.q), k=f(self.k), v=f(self.v), a=f(self.a), b=f(self.b), log_alpha=f(self.log_alpha),
                    initial_state=f(self.initial_state), cu_seqlens=cu)


def make_dplr(seed: int, B: int, T: int, H: int, dtype: str, la_mode: str = "scaled", la_scale: float = 0.1,
              s0_std: float = 0.0, num_seqs: Optional[int] = None, lowrank: str = "tied", ab_scale: float = 1.0,
              device="cuda", dk: int = D, dv: int = D) -> DplrInputs:
    """Inputs of the general DPLR recurrence. q, k, v and log_alpha are drawn as in
    ``make_prefill`` (same draw order up to log_alpha). The low-rank pair:
      "tied": u ~ N(0, 1) L2-normalised per (token, head) and rounded to the compute
              dtype gives b = u; a = -2^-j b with 2^-j = sigmoid(N(0, 1)) rounded to a
              power of two (j >= 1), which is exact in the compute dtype. The
              transition Diag(alpha) - 2^-j b b^T is then symmetric with eigenvalues
              in (-1, 1] whatever the rounding, so the state stays bounded at any length.
      "free": a, b ~ ab_scale N(0, 1/dk) independently (short sequences only).
    Host draws in the order: cut points, q, k, v, log-decay normals, slow-channel
    choice (mixed), then u and the strength normals (tied) or a and b (free), then the
    initial state."""
    dr = HostDraws(seed)
    cu = None
    if num_seqs is not None:
        assert B == 1
        cu = torch.from_numpy(_host_composition(np.random.default_rng(dr.child()), T, num_seqs)).to(device)
    shape_k, shape_v = (B, T, H, dk), (B, T, H, dv)
    nk, nv = B * T * H * dk, B * T * H * dv
    q = _to_device(dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk)), shape_k, dtype, device)
    k = _to_device(dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk)), shape_k, dtype, device)
    v = _to_device(dr.fill(nv, _h_normal), shape_v, dtype, device)
    if la_mode == "scaled":
        la = dr.fill(nk, lambda r, c: -la_scale * _h_softplus(r.standard_normal(c)))
    elif la_mode == "mixed":
        la = dr.fill(nk, lambda r, c: -_h_softplus(r.standard_normal(c))).reshape(B * T, H, dk)
        rs = np.random.default_rng(dr.child())
        for h in range(H):
            slow = rs.permutation(dk)[: dk // 2]
            la[:, h, slow] = np.float32(-1e-3)
        la = la.reshape(-1)
    else:
        raise ValueError(la_mode)
    log_alpha = _to_device(la, shape_k, "fp32", device)
    if lowrank == "tied":
        b = _to_device(dr.fill(nk, lambda r, c: _h_unit_rows(r, c, dk)), shape_k, dtype, device)
        # 2^-j = sigmoid(z) rounded to a power of two, j >= 1: exact in every dtype
        j = dr.fill(B * T * H, lambda r, c: np.maximum(np.round(-np.log2(_h_sigmoid(r.standard_normal(c)))), 1.0))
        scale = torch.from_numpy(-np.exp2(-j.astype(np.float64)).astype(np.float32)).view(B, T, H, 1).to(device)
        a = (scale * b.float()).to(b.dtype)
    elif lowrank == "free":
        sd = ab_scale / dk ** 0.5
        a = _to_device(dr.fill(nk, lambda r, c: sd * r.standard_normal(c)), shape_k, dtype, device)
        b = _to_device(dr.fill(nk, lambda r, c: sd * r.standard_normal(c)), shape_k, dtype, device)
    else:
        raise ValueError(lowrank)
    N = B if cu is None else cu.numel() - 1
    s0 = None
    if s0_std > 0:
        s0 = _to_device(dr.fill(N * H * dk * dv, lambda r, c: s0_std * r.standard_normal(c)), (N, H, dk, dv), "fp32",
                        device)
    return DplrInputs(q.contiguous(), k.contiguous(), v.contiguous(), a.contiguous(), b.contiguous(),
                      log_alpha.contiguous(), s0, cu, dtype,
                      dict(seed=seed, la_mode=la_mode, la_scale=la_scale, lowrank=lowrank))
