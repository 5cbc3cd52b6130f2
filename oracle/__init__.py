"""CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product package.

Contents
--------
``forward`` / ``decode_step``
    The sequential fp64 recurrence in C (``kda_oracle.c``), through ctypes.
``reference``
    Plain NumPy forms used to pin the C oracle: the explicit product of dense
    transition matrices, the textbook DeltaNet and Gated DeltaNet updates.
``chunked``
    The chunkwise (WY / UT) form in fp64 and an emulation of the in-chunk decay
    factoring, each checked against the sequential recurrence.
``exact``
    Exact rational evaluation of the dense form for the golden fixtures.
``fused``
    The layer's prologue (q, k L2 normalisation, gate and beta activations) and
    epilogue (output RMSNorm and gate) around the recurrence.
``dplr_forward``
    The general diagonal-plus-low-rank recurrence
    S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T, sequential fp64 in C; the
    comparison point for KDA's chunk kernel. ``reference`` and ``chunked`` hold its
    dense product, gated-linear-attention and chunkwise forms.
``backward``
    Gradients of the recurrence with respect to q, k, v, log_alpha, beta and the
    initial state, by reverse mode through the sequential fp64 form in C.

Parity status: every function here is pinned by a ``-m "not gpu"`` test; none is
"parity unpinned".
"""
from .build import build_oracle, oracle_lib_path
from .seq import backward, decode_step, dplr_forward, forward, load_library

__all__ = ["build_oracle", "oracle_lib_path", "forward", "decode_step", "backward", "dplr_forward", "load_library"]
