"""Python binding of libkda.so: argument marshalling only.

Every step of the computation runs in the HIP library; this module checks that
torch tensors have the layout the C ABI documents (include/kda.h), passes their
device pointers and the current HIP stream, and turns status codes into
exceptions. PyTorch supplies device memory and streams, nothing else. Importing
this module fails loudly when the library is missing: there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_BF16 = 0
KDA_FP32 = 1
KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_DEVICE = -4

EXPORTS = ("kda_abi_version", "kda_status_string", "kda_last_error", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_fused", "kda_decode_step_fused",
           "kda_output_norm_gate", "kda_timing_enable", "kda_timing_read", "kda_chunk_bwd_workspace_size",
           "kda_chunk_bwd", "kda_dplr_chunk_fwd_workspace_size", "kda_dplr_chunk_fwd",
           "kda_chunk_fwd_fused_workspace_size", "kda_chunk_fwd_noalloc")

KERNEL_NAMES = ("plan", "intra", "inter", "decode", "outnorm", "bwd_local", "bwd_state",
                "bwd_chunk", "seg_first", "seg_scan", "seg_second")  # KDA_KERNEL_* ids


class Fusion(ctypes.Structure):
    """kda_fusion (include/kda.h): the layer prologue and epilogue around the
    recurrence. Build one with ``fusion()``."""
    _fields_ = [("normalize_qk", ctypes.c_int), ("qk_eps", ctypes.c_float),
                ("gate_preactivation", ctypes.c_int), ("beta_preactivation", ctypes.c_int),
                ("out_gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("gate_kind", ctypes.c_int), ("prefill_path", ctypes.c_int)]


KDA_GATE_CHANNEL, KDA_GATE_HEAD, KDA_GATE_NONE = 0, 1, 2
KDA_PATH_AUTO, KDA_PATH_RECORD, KDA_PATH_SINGLE_PASS, KDA_PATH_RECORD_SEGMENTED = 0, 1, 2, 3
_PATHS = {"auto": KDA_PATH_AUTO, "record": KDA_PATH_RECORD, "single": KDA_PATH_SINGLE_PASS,
          "segmented": KDA_PATH_RECORD_SEGMENTED}


class KdaError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{detail} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkda.so is not built at {LIB_PATH}; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_abi_version.restype = I
    lib.kda_abi_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [I]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_chunk_fwd_workspace_size.restype = Z
    lib.kda_chunk_fwd_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.kda_decode_step.restype = I
    lib.kda_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.kda_chunk_fwd_fused_workspace_size.restype = Z
    lib.kda_chunk_fwd_fused_workspace_size.argtypes = [I, I, I, I, I, I, P]
    lib.kda_chunk_fwd_fused.restype = I
    lib.kda_chunk_fwd_fused.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P, P, Z, P]
    lib.kda_chunk_fwd_noalloc.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P]
    lib.kda_decode_step_fused.restype = I
    lib.kda_decode_step_fused.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.kda_output_norm_gate.restype = I
    lib.kda_output_norm_gate.argtypes = [P, P, P, P, ctypes.c_int64, I, ctypes.c_float, I, P]
    lib.kda_chunk_bwd_workspace_size.restype = Z
    lib.kda_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I]
    lib.kda_chunk_bwd.restype = I
    lib.kda_chunk_bwd.argtypes = [P, P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.kda_dplr_chunk_fwd_workspace_size.restype = Z
    lib.kda_dplr_chunk_fwd_workspace_size.argtypes = [I, I, I, I, I]
    lib.kda_dplr_chunk_fwd.restype = I
    lib.kda_dplr_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.kda_timing_enable.restype = I
    lib.kda_timing_enable.argtypes = [I]
    lib.kda_timing_read.restype = I
    lib.kda_timing_read.argtypes = [P, P, I]
    return lib


lib = _load()


def _check(status):
    if status != KDA_OK:
        raise KdaError(status, lib.kda_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _path_code(path):
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}, got {path!r}")
    return _PATHS[path]


def workspace_size(B, T, H, num_seqs=0, chunk=64, dtype=KDA_BF16, path="auto") -> int:
    """Workspace bytes of ``chunk_fwd`` on ``path`` (kda_prefill_path: "auto", "record",
    "single" or "segmented"; only bf16 with 64-token chunks has a choice)."""
    code = _path_code(path)
    if code == KDA_PATH_AUTO:
        return int(lib.kda_chunk_fwd_workspace_size(B, T, H, num_seqs, chunk, dtype))
    f = Fusion()
    f.prefill_path = code
    return int(lib.kda_chunk_fwd_fused_workspace_size(B, T, H, num_seqs, chunk, dtype, ctypes.byref(f)))


def fusion(normalize_qk=True, qk_eps=1e-6, gate_preactivation=True, beta_preactivation=True,
           out_gate=None, norm_weight=None, norm_eps=1e-6, path="auto"):
    """A kda_fusion for ``chunk_fwd`` / ``decode_step``. ``out_gate`` (o's shape and
    dtype) and ``norm_weight`` (fp32 [128]) are device tensors or None; the returned
    object keeps them referenced while it lives. ``path`` selects the prefill kernels
    (see ``workspace_size``)."""
    if out_gate is not None:
        if norm_weight is None:
            raise ValueError("out_gate needs norm_weight")
        _need(norm_weight, "norm_weight", torch.float32, (norm_weight.numel(),))
        if not out_gate.is_contiguous():
            raise ValueError("out_gate must be contiguous")
    f = Fusion(int(bool(normalize_qk)), float(qk_eps), int(bool(gate_preactivation)), int(bool(beta_preactivation)),
               None if out_gate is None else out_gate.data_ptr(),
               None if out_gate is None else norm_weight.data_ptr(), float(norm_eps), KDA_GATE_CHANNEL,
               _path_code(path))
    f._keep = (out_gate, norm_weight)
    return f


def _gate_kind(log_alpha, lead, dk):
    """The kda_gate of a log_alpha argument: [..., dk] per channel, [...] per
    (token, head), None for no decay."""
    if log_alpha is None:
        return KDA_GATE_NONE
    if tuple(log_alpha.shape) == tuple(lead):
        _need(log_alpha, "log_alpha", torch.float32, lead)
        return KDA_GATE_HEAD
    _need(log_alpha, "log_alpha", torch.float32, tuple(lead) + (dk,))
    return KDA_GATE_CHANNEL


def _with_gate(f, gate, path="auto"):
    """The Fusion to pass for ``gate`` and ``path``: ``f`` with its gate_kind (and a
    non-default path) set, a plain one when only the gate or the path differs from the
    default, or None for the plain call."""
    code = _path_code(path)
    if f is None and gate == KDA_GATE_CHANNEL and code == KDA_PATH_AUTO:
        return None
    if f is None:
        f = fusion(normalize_qk=False, gate_preactivation=False, beta_preactivation=False)
    f.gate_kind = gate
    if code != KDA_PATH_AUTO:
        f.prefill_path = code
    return f


def _check_out_gate(f, o):
    if f is not None and f.out_gate:
        g = f._keep[0]
        if g.dtype != o.dtype or tuple(g.shape) != tuple(o.shape) or g.device != o.device:
            raise ValueError(f"out_gate must match o: {tuple(o.shape)} {o.dtype}")


def _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens, output_final_state, o, final_state):
    """Checks the prefill tensors; returns (B, T, H, dk, dv, dtype code, N, o, final_state)
    with o and final_state allocated when not given."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dcode = _dtype_code(q)
    _need(q, "q", dt, (B, T, H, dk))
    _need(k, "k", dt, (B, T, H, dk))
    _need(v, "v", dt, (B, T, H, dv))
    _need(beta, "beta", torch.float32, (B, T, H))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    else:
        _need(o, "o", dt, (B, T, H, dv))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    return B, T, H, dk, dv, dcode, N, o, final_state


def chunk_fwd(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, chunk=64,
              output_final_state=True, o=None, final_state=None, workspace=None, fusion=None, path="auto"):
    """Chunked KDA prefill through ``kda_chunk_fwd`` (``kda_chunk_fwd_fused`` when
    ``fusion`` is given, see ``fusion()``, the gate is not per channel or ``path`` is
    "record").

    q, k: [B, T, H, 128]; v: [B, T, H, 128] (bf16 or fp32, all the same);
    log_alpha: [B, T, H, 128] fp32 (KDA), [B, T, H] fp32 (one decay per token and
    head: Gated DeltaNet) or None (no decay: DeltaNet); beta: [B, T, H] fp32;
    initial_state: [N, H, 128, 128] fp32 or None; cu_seqlens: int32 [N+1] device
    tensor (B must be 1) or None. Returns (o, final_state or None).
    """
    B, T, H, dk, dv, dcode, N, o, final_state = _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                                              output_final_state, o, final_state)
    gate = _gate_kind(log_alpha, (B, T, H), dk)
    fusion = _with_gate(fusion, gate, path)
    ws_bytes = 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        ws_bytes = workspace.numel()
    if fusion is None:
        _check(lib.kda_chunk_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            N if cu_seqlens is not None else 0, _ptr(o), _ptr(final_state), B, T, H, dk, dv, chunk, dcode,
            _ptr(workspace), ws_bytes, _stream(q.device)))
    else:
        _check_out_gate(fusion, o)
        _check(lib.kda_chunk_fwd_fused(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            N if cu_seqlens is not None else 0, _ptr(o), _ptr(final_state), B, T, H, dk, dv, chunk, dcode,
            ctypes.byref(fusion), _ptr(workspace), ws_bytes, _stream(q.device)))
    return o, final_state


#: bytes of the static scratch behind ``chunk_fwd_noalloc`` (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, chunk=64,
                      output_final_state=True, o=None, final_state=None):
    """Chunked KDA prefill through ``kda_chunk_fwd_noalloc``: the library allocates
    nothing (its scratch is a static per-device array of NOALLOC_SCRATCH_BYTES).
    Tensors as in ``chunk_fwd`` with a per-channel log_alpha; pass ``o`` and
    ``final_state`` to keep this call free of allocations on the Python side too.
    Calls that overlap on one GPU race on the shared scratch."""
    B, T, H, dk, dv, dcode, N, o, final_state = _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                                              output_final_state, o, final_state)
    _need(log_alpha, "log_alpha", torch.float32, (B, T, H, dk))
    _check(lib.kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        N if cu_seqlens is not None else 0, _ptr(o), _ptr(final_state), B, T, H, dk, dv, chunk, dcode,
        _stream(q.device)))
    return o, final_state


def bwd_workspace_size(B, T, H, num_seqs=0, dtype=KDA_BF16) -> int:
    return int(lib.kda_chunk_bwd_workspace_size(B, T, H, num_seqs, dtype))


def chunk_bwd(q, k, v, log_alpha, beta, grad_o, initial_state=None, grad_final_state=None, cu_seqlens=None,
              workspace=None, want_grad_initial_state=True):
    """Gradients of the plain recurrence through ``kda_chunk_bwd``: for the loss
    sum <o, grad_o> + sum <final_state, grad_final_state>, with respect to q, k, v,
    log_alpha, beta and initial_state. Shapes as ``chunk_fwd`` (per-channel
    log_alpha); grad_o has o's shape and dtype; grad_final_state is fp32
    [N, H, 128, 128] or None. Returns a dict of tensors: grad_q, grad_k, grad_v
    (input dtype), grad_log_alpha, grad_beta (fp32) and grad_initial_state (fp32,
    or None when not wanted).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dcode = _dtype_code(q)
    _need(q, "q", dt, (B, T, H, dk))
    _need(k, "k", dt, (B, T, H, dk))
    _need(v, "v", dt, (B, T, H, dv))
    _need(log_alpha, "log_alpha", torch.float32, (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(grad_o, "grad_o", dt, (B, T, H, dv))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if grad_final_state is not None:
        _need(grad_final_state, "grad_final_state", torch.float32, (N, H, dk, dv))
    out = {"grad_q": torch.empty_like(q), "grad_k": torch.empty_like(k), "grad_v": torch.empty_like(v),
           "grad_log_alpha": torch.empty_like(log_alpha), "grad_beta": torch.empty_like(beta),
           "grad_initial_state": (torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
                                  if want_grad_initial_state else None)}
    ws_bytes = 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        ws_bytes = workspace.numel()
    _check(lib.kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        N if cu_seqlens is not None else 0, _ptr(grad_o), _ptr(grad_final_state), _ptr(out["grad_q"]),
        _ptr(out["grad_k"]), _ptr(out["grad_v"]), _ptr(out["grad_log_alpha"]), _ptr(out["grad_beta"]),
        _ptr(out["grad_initial_state"]), B, T, H, dk, dv, dcode, _ptr(workspace), ws_bytes, _stream(q.device)))
    return out


def dplr_workspace_size(B, T, H, num_seqs=0, dtype=KDA_BF16) -> int:
    return int(lib.kda_dplr_chunk_fwd_workspace_size(B, T, H, num_seqs, dtype))


def dplr_chunk_fwd(q, k, v, a, b, log_alpha, initial_state=None, cu_seqlens=None, output_final_state=True,
                   o=None, final_state=None, workspace=None, chunk=64):
    """Chunked forward of the general DPLR recurrence
    S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, through
    ``kda_dplr_chunk_fwd``. q, k, a, b: [B, T, H, 128]; v: [B, T, H, 128] (bf16 or
    fp32, all the same); log_alpha: [B, T, H, 128] fp32; initial_state,
    cu_seqlens as ``chunk_fwd``. Returns (o, final_state or None)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dcode = _dtype_code(q)
    for t, name in ((q, "q"), (k, "k"), (a, "a"), (b, "b")):
        _need(t, name, dt, (B, T, H, dk))
    _need(v, "v", dt, (B, T, H, dv))
    _need(log_alpha, "log_alpha", torch.float32, (B, T, H, dk))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    else:
        _need(o, "o", dt, (B, T, H, dv))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    ws_bytes = 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        ws_bytes = workspace.numel()
    _check(lib.kda_dplr_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), _ptr(initial_state), _ptr(cu_seqlens),
        N if cu_seqlens is not None else 0, _ptr(o), _ptr(final_state), B, T, H, dk, dv, chunk, dcode,
        _ptr(workspace), ws_bytes, _stream(q.device)))
    return o, final_state


def decode_step(q, k, v, log_alpha, beta, state, o=None, fusion=None):
    """One decode step through ``kda_decode_step`` (``kda_decode_step_fused`` when
    ``fusion`` is given or the gate is not per channel); ``state`` [N, H, 128, 128]
    fp32 is updated in place. q, k, v: [N, H, 128]; log_alpha: [N, H, 128] fp32,
    [N, H] fp32 or None (as in ``chunk_fwd``); beta: [N, H] fp32.
    Returns o [N, H, 128]."""
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    dcode = _dtype_code(q)
    _need(q, "q", dt, (N, H, dk))
    _need(k, "k", dt, (N, H, dk))
    _need(v, "v", dt, (N, H, dv))
    gate = _gate_kind(log_alpha, (N, H), dk)
    _need(beta, "beta", torch.float32, (N, H))
    _need(state, "state", torch.float32, (N, H, dk, dv))
    fusion = _with_gate(fusion, gate)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=q.device)
    else:
        _need(o, "o", dt, (N, H, dv))
    if fusion is None:
        _check(lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state), _ptr(o),
                                   N, H, dk, dv, dcode, _stream(q.device)))
    else:
        _check_out_gate(fusion, o)
        _check(lib.kda_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state),
                                         _ptr(o), N, H, dk, dv, dcode, ctypes.byref(fusion), _stream(q.device)))
    return o


def output_norm_gate(o, gate, weight, eps=1e-6, out=None):
    """``kda_output_norm_gate``: out = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate)
    over the last axis (128). o, gate, out: same shape and dtype; weight: fp32 [128].
    ``out`` may be ``o`` (in place)."""
    dcode = _dtype_code(o)
    dv = o.shape[-1]
    _need(o, "o", o.dtype, tuple(o.shape))
    _need(gate, "gate", o.dtype, tuple(o.shape))
    _need(weight, "weight", torch.float32, (dv,))
    if out is None:
        out = torch.empty_like(o)
    else:
        _need(out, "out", o.dtype, tuple(o.shape))
    rows = o.numel() // dv
    _check(lib.kda_output_norm_gate(_ptr(o), _ptr(gate), _ptr(weight), _ptr(out), rows, dv, float(eps), dcode,
                                    _stream(o.device)))
    return out


def timing_enable(on: bool = True):
    """Start (and clear) or stop per-kernel event timing in the library."""
    _check(lib.kda_timing_enable(1 if on else 0))


def timing_read():
    """Per-kernel totals since the last enable/read: {name: (total_ms, launches)}."""
    n = len(KERNEL_NAMES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _check(lib.kda_timing_read(ms, cnt, n))
    return {KERNEL_NAMES[i]: (ms[i], cnt[i]) for i in range(n)}
