"""ctypes front end of the sequential fp64 oracle (``kda_oracle.c``).

Test infrastructure only. Inputs are float32 NumPy arrays holding the exact
values the GPU receives (bf16 and fp32 values are both exact in float32, and
float32 -> float64 is exact); all arithmetic is fp64 in C.
"""
import ctypes
import os

import numpy as np

from .build import build_oracle, oracle_lib_path, oracle_source_path

_lib = None


def load_library(path=None):
    """Load liboracle.so, compiling it first if it is not there. With ``path``, load
    that build of the oracle source instead (not cached)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    own = path is None
    if own:
        path = oracle_lib_path()
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(oracle_source_path()):
            build_oracle()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.kda_oracle_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, I, I, P, P, I]
    lib.kda_oracle_forward.restype = I
    lib.kda_oracle_forward_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, I, I, I, P, P, I, I, D]
    lib.kda_oracle_forward_ex.restype = I
    lib.kda_oracle_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I]
    lib.kda_oracle_decode_step.restype = I
    lib.kda_oracle_decode_step_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D]
    lib.kda_oracle_decode_step_ex.restype = I
    lib.kda_oracle_backward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, P, P, I]
    lib.kda_oracle_backward.restype = I
    lib.dplr_oracle_forward.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, I, I, I, P, P, I]
    lib.dplr_oracle_forward.restype = I
    lib.kda_oracle_abi_version.restype = I
    if own:
        _lib = lib
    return lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# prologue flags of the C oracle (see kda_oracle.c)
NORM_QK, GATE_PRE, BETA_PRE = 1, 2, 4


def prologue_flags(normalize_qk=False, gate_preactivation=False, beta_preactivation=False):
    return (NORM_QK if normalize_qk else 0) | (GATE_PRE if gate_preactivation else 0) | \
        (BETA_PRE if beta_preactivation else 0)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None,
            heads=None, cols=None, num_threads=None, want_o=True, want_final=True, lib=None,
            flags=0, qk_eps=0.0):
    """Sequential fp64 KDA over every sequence.

    q, k, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H].
    Without ``cu_seqlens`` each of the B rows is one sequence. With it, B must be
    1 and sequence n is tokens [cu_seqlens[n], cu_seqlens[n+1]).
    initial_state: [N, H, dk, dv] or None (zeros).
    heads: list of head indices to compute (default all); cols: (c0, c1) value
    columns to compute (default all). Returns (o, final):
    o [B, T, len(heads), c1-c0] float64, final [N, len(heads), dk, c1-c0] float64.
    ``lib`` substitutes another build of the same C source (used by the test that
    plants mistakes in copies of the oracle). ``flags`` (from ``prologue_flags``)
    and ``qk_eps`` select the prologue on raw inputs: q, k L2 normalisation,
    log_alpha = -softplus(preactivation), beta = sigmoid(preactivation).
    """
    lib = lib or load_library()
    q, k, v, log_alpha, beta = map(_f32, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and log_alpha.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is None:
        starts = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1
        starts = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        assert starts[0] == 0 and starts[-1] == T
    N = len(starts) - 1
    if heads is None:
        heads_arr = None
        nh = H
    else:
        heads_arr = np.ascontiguousarray(np.asarray(heads), dtype=np.int32)
        assert heads_arr.min() >= 0 and heads_arr.max() < H
        nh = len(heads_arr)
    c0, c1 = (0, dv) if cols is None else cols
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, nh, c1 - c0), dtype=np.float64) if want_o else None
    fin = np.zeros((N, nh, dk, c1 - c0), dtype=np.float64) if want_final else None
    rc = lib.kda_oracle_forward_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0), _ptr(starts),
        N, H, dk, dv, _ptr(heads_arr), nh, c0, c1, _ptr(o), _ptr(fin),
        num_threads or default_threads(), int(flags), float(qk_eps))
    if rc != 0:
        raise ValueError(f"kda_oracle_forward rejected its arguments (status {rc})")
    return o, fin


def decode_step(q, k, v, log_alpha, beta, state, num_threads=None, flags=0, qk_eps=0.0):
    """One in-place fp64 decode step. q, k, log_alpha: [N, H, dk]; v: [N, H, dv];
    beta: [N, H]; state: [N, H, dk, dv] float64 (updated in place). Returns o
    [N, H, dv] float64."""
    lib = load_library()
    q, k, v, log_alpha, beta = map(_f32, (q, k, v, log_alpha, beta))
    assert state.dtype == np.float64 and state.flags.c_contiguous
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert state.shape == (N, H, dk, dv)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.kda_oracle_decode_step_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state), _ptr(o),
        N, H, dk, dv, num_threads or default_threads(), int(flags), float(qk_eps))
    if rc != 0:
        raise ValueError(f"kda_oracle_decode_step rejected its arguments (status {rc})")
    return o


def backward(q, k, v, log_alpha, beta, d_o=None, initial_state=None, d_final=None, cu_seqlens=None,
             num_threads=None, lib=None):
    """fp64 gradients of L = sum <o, d_o> + sum <final_state, d_final> with respect to
    q, k, v, log_alpha, beta and initial_state, by reverse-mode through the sequential
    recurrence (``kda_oracle_backward``).

    Shapes as ``forward``; d_o: [B, T, H, dv] (None: zeros); d_final: [N, H, dk, dv]
    (None: zeros). Returns a dict of float64 arrays: dq, dk, dlog_alpha [B, T, H, dk],
    dv [B, T, H, dv], dbeta [B, T, H], d_initial [N, H, dk, dv].
    """
    lib = lib or load_library()
    q, k, v, log_alpha, beta = map(_f32, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and log_alpha.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is None:
        starts = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1
        starts = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        assert starts[0] == 0 and starts[-1] == T
    N = len(starts) - 1
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    df = None if d_final is None else np.ascontiguousarray(d_final, dtype=np.float64)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    if df is not None:
        assert df.shape == (N, H, dk, dv)
    do = None if d_o is None else _f32(d_o)
    if do is not None:
        assert do.shape == v.shape
    out = {name: np.zeros(shape, dtype=np.float64) for name, shape in (
        ("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("dlog_alpha", q.shape), ("dbeta", beta.shape),
        ("d_initial", (N, H, dk, dv)))}
    rc = lib.kda_oracle_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0), _ptr(starts), N, H, dk, dv,
        _ptr(do), _ptr(df), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
        _ptr(out["dbeta"]), _ptr(out["d_initial"]), num_threads or default_threads())
    if rc != 0:
        raise ValueError(f"kda_oracle_backward rejected its arguments (status {rc})")
    return out


def dplr_forward(q, k, v, a, b, log_alpha, initial_state=None, cu_seqlens=None, heads=None, cols=None,
                 num_threads=None, want_o=True, want_final=True, lib=None):
    """Sequential fp64 general-DPLR recurrence over every sequence:

        S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T ,   o_t = S_t^T q_t

    (the comparison point of the GeekNews "Kimi Linear" summary, section "일반 DPLR보다
    줄어든 연산량"). q, k, a, b, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; the rest
    as ``forward``. Returns (o, final) in float64.
    """
    lib = lib or load_library()
    q, k, v, a, b, log_alpha = map(_f32, (q, k, v, a, b, log_alpha))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for x in (k, a, b, log_alpha):
        assert x.shape == q.shape
    assert v.shape == (B, T, H, dv)
    if cu_seqlens is None:
        starts = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1
        starts = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        assert starts[0] == 0 and starts[-1] == T
    N = len(starts) - 1
    if heads is None:
        heads_arr, nh = None, H
    else:
        heads_arr = np.ascontiguousarray(np.asarray(heads), dtype=np.int32)
        assert heads_arr.min() >= 0 and heads_arr.max() < H
        nh = len(heads_arr)
    c0, c1 = (0, dv) if cols is None else cols
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, nh, c1 - c0), dtype=np.float64) if want_o else None
    fin = np.zeros((N, nh, dk, c1 - c0), dtype=np.float64) if want_final else None
    rc = lib.dplr_oracle_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), _ptr(s0), _ptr(starts),
        N, H, dk, dv, _ptr(heads_arr), nh, c0, c1, _ptr(o), _ptr(fin), num_threads or default_threads())
    if rc != 0:
        raise ValueError(f"dplr_oracle_forward rejected its arguments (status {rc})")
    return o, fin
