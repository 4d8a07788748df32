"""Exact, IO-aware, tiled attention forward for MI355X (gfx950).

The compute path is the C-ABI library libfa.so (hand-written HIP kernels);
`fwd` below is a thin ctypes binding that marshals torch device tensors into it.
"""
from .fa import fwd, fwd_strided, version, status_str, lib_path  # noqa: F401
