"""Kimi Delta Attention (KDA) token mixer for AMD MI355X (gfx950).

The computation lives in ``libkda.so`` (hand-written HIP kernels behind the C ABI
of ``include/kda.h``); ``kda`` is its Python binding. ``inputs`` draws seeded
synthetic workloads and holds no arithmetic of the method.

``chunk_fwd``, ``decode_step`` and ``workspace_size`` are loaded on first use, so
that ``inputs`` can be imported on machines without the built library.
"""

__all__ = ["chunk_fwd", "decode_step", "workspace_size", "KdaError"]


def __getattr__(name):
    if name in __all__:
        from . import kda
        return getattr(kda, name)
    raise AttributeError(name)
