"""Fused flash-attention training op for MI355X (gfx950): forward with LSE,
the Delta = rowsum(dO * O) preprocess, the backward with native GQA and
additive masks, and a chunked backward that accumulates fp32 dK/dV over a
cached K/V window. The compute runs in hand-written HIP kernels behind the
C ABI in ``include/fa_train.h``; this package is the Python binding over it.
"""
from __future__ import annotations

__all__ = ["fwd", "bwd_preprocess", "bwd", "bwd_chunked", "bwd_workspace_bytes", "mask_tile_map", "library_path"]


def __getattr__(name):  # the binding (and the HIP library) is loaded on first use
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
