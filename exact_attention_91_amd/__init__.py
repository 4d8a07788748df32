"""Exact, IO-aware, tiled attention for MI355X (gfx950): forward, key-split
forward with a logsumexp combine, sliding-window / local-global forward, and
backward.

The compute path is the C-ABI library libfa.so (hand-written HIP kernels);
the functions below are a thin ctypes binding that marshals torch device
tensors into it.
"""
from .fa import (fwd, fwd_strided, fwd_splitk, lse_combine, splitk_workspace_bytes,  # noqa: F401
                 fwd_window, window_bitmap, bwd, bwd_window, bwd_workspace_bytes,
                 bwd_window_workspace_bytes, version, status_str, lib_path)
