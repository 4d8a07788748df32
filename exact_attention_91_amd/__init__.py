"""Exact, IO-aware, tiled attention forward for MI355X (gfx950).

The compute path is the C-ABI library libfa.so (hand-written HIP kernels);
the functions below are a thin ctypes binding that marshals torch device
tensors into it.
"""
from .fa import (fwd, fwd_strided, fwd_splitk, lse_combine, splitk_workspace_bytes,  # noqa: F401
                 version, status_str, lib_path)
