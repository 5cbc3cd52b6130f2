"""Prologue and epilogue around the KDA recurrence, in fp64 -- test infrastructure.

The Kimi Linear layer (GeekNews "Kimi Linear" summary, section "Kimi Linear 모델
구성") L2-normalises each head's query and key for eigenvalue stability, takes the
per-channel decay from a GDN/Mamba-like decay function of a low-rank projection,
and applies a per-head RMSNorm and a data-dependent output gate before the output
projection. Where the page leaves a step open, the readings are:

  q, k        x / sqrt(sum_i x_i^2 + eps)       per (token, head), eps given by the caller
  log alpha   -softplus(a)                      a = gate pre-activation, per channel
  beta        sigmoid(b)                        b = pre-activation, per (token, head)
  output      o / sqrt(mean_j o_j^2 + eps) * w * sigmoid(z)
                                                per (token, head) over the dv values;
                                                w: [dv] shared by the heads; z: gate
                                                pre-activation with o's layout

The prologue runs inside the C oracle (``seq.forward(..., flags=...)``) so that the
normalised vectors never leave fp64; the epilogue needs whole output rows and is
applied here. Every function is pinned by tests/test_oracle_fused.py.
"""
import numpy as np

from . import seq


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + np.log1p(np.exp(-np.abs(x))), np.log1p(np.exp(np.minimum(x, 0.0))))


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2_normalize(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gate_log_alpha(a):
    return -softplus(a)


def output_norm_gate(o, z, w, eps):
    """RMSNorm over the last axis, times the weight and the sigmoid output gate."""
    o = np.asarray(o, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(w, dtype=np.float64) * sigmoid(z)


def forward(q, k, v, gate, beta_pre, initial_state=None, cu_seqlens=None, out_gate=None, norm_weight=None,
            qk_eps=1e-6, norm_eps=1e-6, heads=None, num_threads=None, want_final=True):
    """The fused layer core on raw inputs: prologue, the sequential recurrence, and
    (when ``out_gate`` is given) the output RMSNorm and gate. Shapes as in
    ``seq.forward``; ``gate`` has log_alpha's shape, ``beta_pre`` beta's,
    ``out_gate`` o's. Returns (o, final) in fp64 for the selected heads."""
    flags = seq.prologue_flags(normalize_qk=True, gate_preactivation=True, beta_preactivation=True)
    o, fin = seq.forward(q, k, v, gate, beta_pre, initial_state, cu_seqlens, heads=heads,
                         num_threads=num_threads, want_final=want_final, flags=flags, qk_eps=qk_eps)
    if out_gate is not None:
        z = np.asarray(out_gate, dtype=np.float64)
        if heads is not None:
            z = z[:, :, list(heads)]
        o = output_norm_gate(o, z, norm_weight, norm_eps)
    return o, fin


def decode_step(q, k, v, gate, beta_pre, state, out_gate=None, norm_weight=None, qk_eps=1e-6, norm_eps=1e-6,
                num_threads=None):
    """One fused decode step (state updated in place); returns o in fp64."""
    flags = seq.prologue_flags(normalize_qk=True, gate_preactivation=True, beta_preactivation=True)
    o = seq.decode_step(q, k, v, gate, beta_pre, state, num_threads=num_threads, flags=flags, qk_eps=qk_eps)
    if out_gate is not None:
        o = output_norm_gate(o, out_gate, norm_weight, norm_eps)
    return o
