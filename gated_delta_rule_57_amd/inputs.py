"""Seeded synthetic inputs for the KDA token mixer.

This module only draws random numbers and shapes them; it holds none of the
recurrence's arithmetic. The tests of the GPU path, the oracle comparisons and
the bench all take their inputs from here. Draws use a ``torch.Generator`` seeded
with ``seed`` on the target device, in a fixed order: cut points (packed
batches), q, k, v, log-decay normals, slow-channel choice (mixed mode), beta
normals, initial state. The same seed on the same device type gives the same
values; the CPU and GPU streams differ.

Distributions (the plainest reading of the workloads the library is measured on):
  q, k      ~ N(0, 1), then L2-normalised per (token, head) in fp32 (the model
              normalises q and k before the mixer; GeekNews "Kimi Linear" summary,
              section "Kimi Linear 모델 구성"), then rounded to the compute dtype
              (bf16: round to nearest even)
  v         ~ N(0, 1), rounded to the compute dtype
  log_alpha = -scale * softplus(N(0, 1)) per channel (fp32). In "mixed" mode a
              seeded half of each head's channels is -1e-3 (slow) and the rest
              -softplus(N(0, 1)) (fast), the same channels at every token
  beta      = sigmoid(N(0, 1)) per (token, head) (fp32)
  S_0       ~ N(0, s0_std) fp32, or None (zeros)
"""
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


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def uniform_composition(g, total: int, parts: int, device) -> torch.Tensor:
    """cu_seqlens of ``parts`` positive lengths summing to ``total``: distinct cut
    points drawn uniformly from [1, total-1] and sorted."""
    cuts = torch.randperm(total - 1, generator=g, device=device)[: parts - 1] + 1
    cuts, _ = torch.sort(cuts)
    z = torch.zeros(1, dtype=cuts.dtype, device=device)
    e = torch.full((1,), total, dtype=cuts.dtype, device=device)
    return torch.cat([z, cuts, e]).to(torch.int32)


def make_prefill(seed: int, B: int, T: int, H: int, dtype: str, chunk: int = 64, la_mode: str = "scaled",
                 la_scale: float = 0.1, s0_std: float = 0.0, num_seqs: Optional[int] = None,
                 cu_seqlens=None, device="cuda", dk: int = D, dv: int = D, gate: str = "channel") -> PrefillInputs:
    """``gate``: "channel" (log_alpha [B, T, H, dk]), "head" (one decay per (token,
    head): log_alpha [B, T, H], drawn like one channel) or "none" (log_alpha None)."""
    g = _gen(seed, device)
    cu = None
    if cu_seqlens is not None:
        assert B == 1
        cu = torch.as_tensor(np.asarray(cu_seqlens), dtype=torch.int32).to(device)
    elif num_seqs is not None:
        assert B == 1
        cu = uniform_composition(g, T, num_seqs, device)
    td = TORCH_DTYPE[dtype]
    q = _unit_rows(_normal(g, (B, T, H, dk), device)).to(td)
    k = _unit_rows(_normal(g, (B, T, H, dk), device)).to(td)
    v = _normal(g, (B, T, H, dv), device).to(td)
    z = _normal(g, (B, T, H, dk) if gate == "channel" else (B, T, H), device)
    if gate == "head":
        assert la_mode == "scaled"
        log_alpha = -la_scale * torch.nn.functional.softplus(z)
    elif gate == "none":
        log_alpha = None
    elif la_mode == "scaled":
        log_alpha = -la_scale * torch.nn.functional.softplus(z)
    elif la_mode == "mixed":
        log_alpha = -torch.nn.functional.softplus(z)
        for h in range(H):
            slow = torch.randperm(dk, generator=g, device=device)[: dk // 2]
            log_alpha[:, :, h, slow] = -1e-3
    else:
        raise ValueError(la_mode)
    beta = torch.sigmoid(_normal(g, (B, T, H), device))
    N = B if cu is None else cu.numel() - 1
    s0 = s0_std * _normal(g, (N, H, dk, dv), device) if s0_std > 0 else None
    return PrefillInputs(q.contiguous(), k.contiguous(), v.contiguous(),
                         None if log_alpha is None else log_alpha.contiguous(), beta.contiguous(),
                         s0, cu, dtype, chunk, dict(seed=seed, la_mode=la_mode, la_scale=la_scale, gate=gate))


def make_cotangents(seed: int, inp: PrefillInputs, final_std: float = 0.1, device="cuda"):
    """Cotangents for a backward call on ``inp``: grad_o ~ N(0, 1) in the input dtype,
    shaped like o, and grad_final_state ~ N(0, final_std^2) fp32 [N, H, dk, dv]
    (None when final_std is 0)."""
    g = _gen(seed + 1000, device)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    grad_o = _normal(g, (B, T, H, dv), device).to(inp.q.dtype).contiguous()
    gf = final_std * _normal(g, (inp.num_seqs, H, dk, dv), device) if final_std > 0 else None
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
    g = _gen(seed, device)
    td = TORCH_DTYPE[dtype]
    s0 = s0_std * _normal(g, (N, H, dk, dv), device)
    qs, ks, vs, las, bs = [], [], [], [], []
    for _ in range(n_steps):
        qs.append(_unit_rows(_normal(g, (N, H, dk), device)).to(td))
        ks.append(_unit_rows(_normal(g, (N, H, dk), device)).to(td))
        vs.append(_normal(g, (N, H, dv), device).to(td))
        las.append(-la_scale * torch.nn.functional.softplus(_normal(g, (N, H, dk), device)))
        bs.append(torch.sigmoid(_normal(g, (N, H), device)))
    st = lambda xs: torch.stack(xs).contiguous()
    return DecodeInputs(s0, st(qs), st(ks), st(vs), st(las), st(bs), dtype)


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
    norm_weight ~ U(0.5, 1.5). Draw order: cut points, q, k, v, gate, beta, out_gate,
    norm_weight, initial state."""
    g = _gen(seed, device)
    cu = None
    if num_seqs is not None:
        assert B == 1
        cu = uniform_composition(g, T, num_seqs, device)
    td = TORCH_DTYPE[dtype]
    q = (qk_scale * _normal(g, (B, T, H, dk), device)).to(td)
    k = (qk_scale * _normal(g, (B, T, H, dk), device)).to(td)
    v = _normal(g, (B, T, H, dv), device).to(td)
    gate = _normal(g, (B, T, H, dk), device) + gate_shift
    beta = _normal(g, (B, T, H), device)
    out_gate = _normal(g, (B, T, H, dv), device).to(td)
    w = 0.5 + torch.rand((dv,), generator=g, device=device, dtype=torch.float32)
    N = B if cu is None else cu.numel() - 1
    s0 = s0_std * _normal(g, (N, H, dk, dv), device) if s0_std > 0 else None
    return RawPrefillInputs(q.contiguous(), k.contiguous(), v.contiguous(), gate.contiguous(), beta.contiguous(),
                            out_gate.contiguous(), w, s0, cu, dtype, chunk)


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
    Draw order: cut points, q, k, v, log-decay normals, slow-channel choice (mixed),
    then u and the strength normals (tied) or a and b (free), then the initial state."""
    g = _gen(seed, device)
    cu = None
    if num_seqs is not None:
        assert B == 1
        cu = uniform_composition(g, T, num_seqs, device)
    td = TORCH_DTYPE[dtype]
    q = _unit_rows(_normal(g, (B, T, H, dk), device)).to(td)
    k = _unit_rows(_normal(g, (B, T, H, dk), device)).to(td)
    v = _normal(g, (B, T, H, dv), device).to(td)
    z = _normal(g, (B, T, H, dk), device)
    if la_mode == "scaled":
        log_alpha = -la_scale * torch.nn.functional.softplus(z)
    elif la_mode == "mixed":
        log_alpha = -torch.nn.functional.softplus(z)
        for h in range(H):
            slow = torch.randperm(dk, generator=g, device=device)[: dk // 2]
            log_alpha[:, :, h, slow] = -1e-3
    else:
        raise ValueError(la_mode)
    if lowrank == "tied":
        b = _unit_rows(_normal(g, (B, T, H, dk), device)).to(td)
        strength = torch.sigmoid(_normal(g, (B, T, H), device))
        j = torch.clamp(torch.round(-torch.log2(strength)), min=1.0)
        a = (-torch.exp2(-j)[..., None] * b.float()).to(td)
    elif lowrank == "free":
        a = (ab_scale / dk ** 0.5 * _normal(g, (B, T, H, dk), device)).to(td)
        b = (ab_scale / dk ** 0.5 * _normal(g, (B, T, H, dk), device)).to(td)
    else:
        raise ValueError(lowrank)
    N = B if cu is None else cu.numel() - 1
    s0 = s0_std * _normal(g, (N, H, dk, dv), device) if s0_std > 0 else None
    return DplrInputs(q.contiguous(), k.contiguous(), v.contiguous(), a.contiguous(), b.contiguous(),
                      log_alpha.contiguous(), s0, cu, dtype,
                      dict(seed=seed, la_mode=la_mode, la_scale=la_scale, lowrank=lowrank))
