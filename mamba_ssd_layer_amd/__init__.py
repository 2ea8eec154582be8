"""mamba_ssd_layer_amd -- the SSD (state space duality) layer forward pass of
Mamba-2 on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C-ABI library
``libssd.so`` (declared in ``include/ssd.h``); this package only marshals torch
tensors into that library.  Importing the package does not load the library:
the first call of ``ssd_chunked_fwd`` / ``ssd_chunked_fwd_varlen`` does, and
raises if it is missing (there is no CPU fallback).
"""
from __future__ import annotations

__all__ = ["ssd_chunked_fwd", "ssd_chunked_fwd_varlen", "ssd_chunked_fwd_intermediates",
           "SSDError", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
