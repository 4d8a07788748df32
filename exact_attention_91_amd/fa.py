"""Thin ctypes binding over libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, and the calls into the library (forward, key-split forward, combine,
backward) on torch's current stream. Every step of the attention runs in the
library's HIP kernels; there is no fallback. If libfa.so is missing, every
call raises.
"""
import contextlib
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
_LIB = None

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2

_I = ctypes.c_int
_VP = ctypes.c_void_p
_LL3 = ctypes.c_longlong * 3
_LLP = ctypes.POINTER(ctypes.c_longlong)


def lib_path() -> str:
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"libfa.so not found at {_LIB_PATH}: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        _LIB = _configure(ctypes.CDLL(_LIB_PATH))
    return _LIB


@contextlib.contextmanager
def using_library(path: str):
    """Inside the with-block every call of this binding goes to the C ABI of
    the library at `path`, another build of the same sources (the LDS-poisoning
    debug build libfa_poison.so in the tests)."""
    global _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first")
    prev = _LIB
    _LIB = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _LIB = prev


def _configure(lib):
    """Declare the argument and result types of every entry point of `lib`."""
    lib.fa_fwd.argtypes = [_VP, _VP, _VP, _VP, _VP] + [_I] * 6 + [ctypes.c_float, _I, _VP]
    lib.fa_fwd.restype = _I
    lib.fa_fwd_strided.argtypes = ([_VP, _VP, _VP, _VP, _VP] + [_I] * 6 +
                                   [ctypes.c_float, _I] + [_LLP] * 4 + [_VP])
    lib.fa_fwd_strided.restype = _I
    lib.fa_fwd_key_groups.argtypes = [_I] * 5
    lib.fa_fwd_key_groups.restype = _I
    lib.fa_fwd_splitk.argtypes = ([_VP, _VP, _VP, _VP, _VP] + [_I] * 6 +
                                  [ctypes.c_float, _I, _I, _VP, ctypes.c_longlong, _VP])
    lib.fa_fwd_splitk.restype = _I
    lib.fa_fwd_splitk_noalloc.argtypes = ([_VP, _VP, _VP, _VP, _VP] + [_I] * 6 +
                                          [ctypes.c_float, _I, _I, _VP])
    lib.fa_fwd_splitk_noalloc.restype = _I
    lib.fa_fwd_splitk_scratch_bytes.argtypes = []
    lib.fa_fwd_splitk_scratch_bytes.restype = ctypes.c_longlong
    lib.fa_fwd_decode.argtypes = ([_VP] * 5 + [_I] * 7 + [ctypes.c_float, _I, _I, _VP,
                                                          ctypes.c_longlong, _VP])
    lib.fa_fwd_decode.restype = _I
    lib.fa_fwd_decode_workspace_bytes.argtypes = [_I] * 5
    lib.fa_fwd_decode_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_fwd_splitk_workspace_bytes.argtypes = [_I] * 5
    lib.fa_fwd_splitk_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_lse_combine.argtypes = [_VP, _VP] + [_I] * 5 + [_VP, _VP, _I, _VP]
    lib.fa_lse_combine.restype = _I
    lib.fa_fwd_window.argtypes = ([_VP] * 5 + [_I] * 6 + [ctypes.c_float, _I, _I, _VP, _VP])
    lib.fa_fwd_window.restype = _I
    lib.fa_window_bitmap.argtypes = [_VP, _I, _I, _VP, ctypes.c_longlong, _VP]
    lib.fa_window_bitmap.restype = _I
    lib.fa_window_bitmap_bytes.argtypes = [_I]
    lib.fa_window_bitmap_bytes.restype = ctypes.c_longlong
    lib.fa_bwd.argtypes = [_VP] * 9 + [_I] * 6 + [ctypes.c_float, _I, _I, _VP,
                                                    ctypes.c_longlong, _VP]
    lib.fa_bwd.restype = _I
    lib.fa_bwd_window.argtypes = ([_VP] * 9 + [_I] * 6 + [ctypes.c_float, _I, _I, _VP, _I,
                                                          _VP, ctypes.c_longlong, _VP])
    lib.fa_bwd_window.restype = _I
    lib.fa_bwd_workspace_bytes.argtypes = [_I] * 6
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_bwd_window_workspace_bytes.argtypes = [_I] * 8
    lib.fa_bwd_window_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_status_str.argtypes = [_I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = _I
    return lib


def version() -> int:
    return int(_lib().fa_version())


def key_groups(B: int, H: int, T: int, D: int, dtype) -> int:
    """Key-range groups per query tile that fwd() uses for these sizes (1 or 2;
    see fa_fwd_key_groups in fa.h). dtype: a torch dtype."""
    code = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16,
            torch.float32: FA_DTYPE_F32}[dtype]
    return int(_lib().fa_fwd_key_groups(B, H, T, D, code))


def status_str(code: int) -> str:
    return _lib().fa_status_str(int(code)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def check_shapes(q, k, v):
    """Raise ValueError unless q is [B, T, H, D] and k, v are both
    [B, T, H_kv, D] with the same B, T and D (the sizes the library reads
    from q alone). Runs before any device check, so it needs no GPU."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D, got {tuple(t.shape)}")
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k and v must have one shape, got {tuple(k.shape)} and "
                         f"{tuple(v.shape)}")
    B, T, _, D = q.shape
    if (k.shape[0], k.shape[1], k.shape[3]) != (B, T, D):
        raise ValueError(f"k/v {tuple(k.shape)} must be [B, T, H_kv, D] with q's "
                         f"B={B}, T={T}, D={D}")


def _check(q, k, v):
    check_shapes(q, k, v)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _raise(rc: int, fn: str):
    if rc != 0:
        raise RuntimeError(f"{fn} failed: {status_str(rc)} (code {rc})")


def fwd(q, k, v, causal: bool = False, scale=None):
    """Attention forward on BNHD-contiguous tensors.

    q: [B, T, H, D], k and v: [B, T, H_kv, D] (bf16, fp16 or fp32, contiguous).
    Returns (o [B, T, H, D] in q's dtype, lse [B, H, T] float32), where lse is
    the natural-log logsumexp of each row's scaled, masked scores.
    """
    _check(q, k, v)
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd needs contiguous [B,T,H,D] tensors; use fwd_strided for views")
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr(), B, H, H_kv, T, D, int(bool(causal)),
                       float(scale), _dtype_code(q), stream)
    _raise(rc, "fa_fwd")
    return o, lse


def fwd_strided(q, k, v, causal: bool = False, scale=None, out_layout: str = "bthd"):
    """Attention forward on views with arbitrary (batch, token, head) strides.

    Tensors are indexed logically as q[b, t, h, :] (pass e.g. x.transpose(1, 2)
    of a [B, H, T, D] tensor); the last dim must have stride 1. `out_layout`
    picks the memory order of o: "bthd" ([B,T,H,D]) or "bhtd" ([B,H,T,D]);
    o is returned as a [B, T, H, D]-indexed view either way.
    """
    _check(q, k, v)
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out_layout == "bthd":
        o = torch.empty((B, T, H, D), dtype=q.dtype, device=q.device)
    elif out_layout == "bhtd":
        o = torch.empty((B, H, T, D), dtype=q.dtype, device=q.device).transpose(1, 2)
    else:
        raise ValueError("out_layout must be 'bthd' or 'bhtd'")
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have unit stride in its last dim")

    def st(t):
        return _LL3(t.stride(0), t.stride(1), t.stride(2))

    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, H, H_kv, T, D, int(bool(causal)),
                               float(scale), _dtype_code(q), st(q), st(k), st(v), st(o),
                               stream)
    _raise(rc, "fa_fwd_strided")
    return o, lse


def splitk_workspace_bytes(B: int, H: int, T: int, D: int, nsplit: int) -> int:
    """Bytes of device workspace fwd_splitk needs (-1 for invalid sizes)."""
    return int(_lib().fa_fwd_splitk_workspace_bytes(B, H, T, D, nsplit))


def fwd_splitk(q, k, v, causal: bool = False, scale=None, nsplit: int = 2, workspace=None):
    """Split-K attention forward (bf16 or fp16, contiguous BNHD): every query
    tile's keys are divided into `nsplit` ranges computed by separate
    work-groups and merged by their logsumexps. Same result as fwd up to
    rounding. `workspace` (optional): a device tensor of at least
    splitk_workspace_bytes(...) bytes; allocated here when None.
    Returns (o, lse) like fwd."""
    _check(q, k, v)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"fwd_splitk takes bfloat16 or float16 inputs, got {q.dtype}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd_splitk needs contiguous [B,T,H,D] tensors")
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = splitk_workspace_bytes(B, H, T, D, nsplit)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = workspace.numel() * workspace.element_size()
    rc = _lib().fa_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, H_kv, T, D, int(bool(causal)),
                              float(scale), _dtype_code(q), int(nsplit),
                              workspace.data_ptr(), nbytes, stream)
    _raise(rc, "fa_fwd_splitk")
    return o, lse


def splitk_scratch_bytes() -> int:
    """Bytes of the library's fixed scratch used by fwd_splitk_noalloc."""
    return int(_lib().fa_fwd_splitk_scratch_bytes())


def fwd_splitk_noalloc(q, k, v, causal: bool = False, scale=None, nsplit: int = 2):
    """fwd_splitk without a workspace: the partials live in the library's fixed
    device scratch (splitk_scratch_bytes()), so the library allocates nothing
    (o and lse are still allocated here). Calls that overlap on one device
    share that scratch and must be ordered on one stream. Returns (o, lse)."""
    _check(q, k, v)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"fwd_splitk_noalloc takes bfloat16 or float16 inputs, got {q.dtype}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd_splitk_noalloc needs contiguous [B,T,H,D] tensors")
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_fwd_splitk_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, H_kv, T, D, int(bool(causal)),
                                      float(scale), _dtype_code(q), int(nsplit), stream)
    _raise(rc, "fa_fwd_splitk_noalloc")
    return o, lse


def decode_workspace_bytes(B: int, H: int, T_q: int, D: int, nsplit: int) -> int:
    """Bytes of device workspace fwd_decode needs (-1 for invalid sizes)."""
    return int(_lib().fa_fwd_decode_workspace_bytes(B, H, T_q, D, nsplit))


def decode_splits(B: int, H_kv: int, H: int, T_q: int, T_k: int) -> int:
    """A key split for fwd_decode: enough parts that the launch has about two
    work-groups per compute unit, each part at least 256 keys, at most 64."""
    units = B * H_kv * -(-(H // H_kv) * T_q // 128)
    want = max(1, -(-512 // max(units, 1)))
    return int(max(1, min(want, T_k // 256, 64)))


def fwd_decode(q, k, v, causal: bool = True, scale=None, nsplit=None, workspace=None):
    """Decode-shaped attention forward (bfloat16 or float16, contiguous):
    q [B, T_q, H, D] holds the last T_q positions of a sequence whose keys and
    values are k, v [B, T_k, H_kv, D] (a key/value cache); under the causal
    mask query i sees keys j <= T_k - T_q + i. The keys are split into `nsplit`
    ranges (decode_splits(...) when None) merged by their logsumexps.
    Returns (o [B, T_q, H, D], lse [B, H, T_q] float32)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D torch tensor")
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k and v must have one shape, got {tuple(k.shape)} and "
                         f"{tuple(v.shape)}")
    B, T_q, H, D = q.shape
    T_k, H_kv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v {tuple(k.shape)} must be [B, T_k, H_kv, D] with q's B={B}, D={D}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("fwd_decode takes bfloat16 or float16 q, k, v of one dtype")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd_decode needs contiguous tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if nsplit is None:
        nsplit = decode_splits(B, H_kv, H, T_q, T_k)
    need = decode_workspace_bytes(B, H, T_q, D, nsplit)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T_q), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, H_kv, T_q, T_k, D, int(bool(causal)),
                              float(scale), _dtype_code(q), int(nsplit), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), stream)
    _raise(rc, "fa_fwd_decode")
    return o, lse


def lse_combine(o_parts, lse_parts, dtype=torch.bfloat16):
    """Merge partial results over disjoint key ranges on the GPU.

    o_parts: float32 [n, B, H, T, D], lse_parts: float32 [n, B, H, T]
    (contiguous). Returns (o [B, T, H, D] in `dtype`, lse [B, H, T] float32)
    with L = ln sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("o_parts and lse_parts must be float32")
    if not (o_parts.is_cuda and lse_parts.is_cuda):
        raise ValueError("o_parts and lse_parts must be GPU tensors")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if o_parts.dim() != 5 or tuple(o_parts.shape[:4]) != tuple(lse_parts.shape):
        raise ValueError("o_parts must be [n, B, H, T, D] and lse_parts [n, B, H, T]")
    n, B, H, T, D = o_parts.shape
    o = torch.empty((B, T, H, D), dtype=dtype, device=o_parts.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=o_parts.device)
    stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    rc = _lib().fa_lse_combine(o_parts.data_ptr(), lse_parts.data_ptr(), n, B, H, T, D,
                               o.data_ptr(), lse.data_ptr(), _dtype_code(o), stream)
    _raise(rc, "fa_lse_combine")
    return o, lse


def window_bitmap(global_tokens, T: int, device):
    """Bitmap of the global tokens for fwd_window (uint8 tensor of
    8*ceil(T/64) bytes on `device`), built by the library's kernel.
    global_tokens: a sequence of ints or a 1-D int32 tensor."""
    g = (global_tokens if isinstance(global_tokens, torch.Tensor)
         else torch.tensor(list(global_tokens), dtype=torch.int32))
    if g.dtype != torch.int32 or g.dim() != 1:
        raise ValueError("global_tokens must be a 1-D int32 tensor or a sequence of ints")
    g = g.to(device).contiguous()
    nbytes = int(_lib().fa_window_bitmap_bytes(T))
    if nbytes < 0:
        raise ValueError(f"bad T {T}")
    bits = torch.empty((max(nbytes, 8),), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    rc = _lib().fa_window_bitmap(g.data_ptr() if g.numel() else None, g.numel(), T,
                                 bits.data_ptr(), bits.numel(), stream)
    _raise(rc, "fa_window_bitmap")
    return bits


def fwd_window(q, k, v, window: int, global_tokens=None, causal: bool = False, scale=None,
               global_bits=None):
    """Sliding-window / local-global attention forward (bfloat16 or float16,
    contiguous BNHD): key j visible to query i iff |i - j| <= window or j is a
    global token, and j <= i when causal. The global tokens are given either
    as `global_tokens` (a sequence of ints or an int32 tensor; the bitmap is
    built for this call) or as a prebuilt `global_bits` from window_bitmap.
    Returns (o, lse) like fwd."""
    _check(q, k, v)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"fwd_window takes bfloat16 or float16 inputs, got {q.dtype}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd_window needs contiguous [B,T,H,D] tensors")
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if global_tokens is not None and global_bits is not None:
        raise ValueError("give global_tokens or global_bits, not both")
    if global_tokens is not None:
        global_bits = window_bitmap(global_tokens, T, q.device)
    if global_bits is not None and global_bits.numel() * global_bits.element_size() < \
            int(_lib().fa_window_bitmap_bytes(T)):
        raise ValueError("global_bits is smaller than window_bitmap builds for this T")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, H_kv, T, D, int(bool(causal)), float(scale),
                              _dtype_code(q), int(window),
                              None if global_bits is None else global_bits.data_ptr(), stream)
    _raise(rc, "fa_fwd_window")
    return o, lse


def bwd_workspace_bytes(B: int, H: int, H_kv: int, T: int, D: int, head_split: int = 0) -> int:
    """Bytes of device workspace bwd needs (-1 for invalid sizes)."""
    return int(_lib().fa_bwd_workspace_bytes(B, H, H_kv, T, D, head_split))


def bwd_window_workspace_bytes(B: int, H: int, H_kv: int, T: int, D: int, window: int,
                               n_global: int, head_split: int = 0) -> int:
    """Bytes of device workspace bwd_window uses to split the far queries of
    up to n_global global tokens (-1 for invalid sizes)."""
    return int(_lib().fa_bwd_window_workspace_bytes(B, H, H_kv, T, D, int(window),
                                                    int(n_global), head_split))


def _bwd_args(q, k, v, o, lse, dout, scale, head_split, workspace, need=None):
    _check(q, k, v)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"the backward takes bfloat16 or float16 inputs, got {q.dtype}")
    B, T, H, D = q.shape
    for name, t, shape, dt in (("o", o, q.shape, q.dtype), ("dout", dout, q.shape, q.dtype),
                               ("lse", lse, (B, H, T), torch.float32)):
        if not isinstance(t, torch.Tensor) or t.device != q.device:
            raise ValueError(f"{name} must be a tensor on {q.device}")
        if tuple(t.shape) != tuple(shape) or t.dtype != dt:
            raise ValueError(f"{name} must be {dt} of shape {tuple(shape)}, got "
                             f"{t.dtype} {tuple(t.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        if not t.is_contiguous():
            raise ValueError(f"the backward needs contiguous tensors ({name} is not)")
    H_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if need is None:
        need = bwd_workspace_bytes(B, H, H_kv, T, D, head_split)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, dout) + grads]
    return (ptrs, (B, H, H_kv, T, D), float(scale), workspace, grads)


def bwd_window(q, k, v, o, lse, dout, window: int, global_tokens=None, causal: bool = False,
               scale=None, global_bits=None, workspace=None, head_split: int = 0,
               n_global=None):
    """Backward of fwd_window (same window, global tokens, causal, scale; o and
    lse from fwd_window). Returns (dq, dk, dv). When `workspace` is None it is
    sized by bwd_window_workspace_bytes for n_global tokens: len(global_tokens),
    or the bits set in global_bits when n_global is not given (a device sync)."""
    if global_tokens is not None and global_bits is not None:
        raise ValueError("give global_tokens or global_bits, not both")
    B, T, H, D = q.shape
    need = None
    if workspace is None and (global_tokens is not None or global_bits is not None):
        if n_global is None:
            if global_tokens is not None:
                n_global = len({int(t) for t in global_tokens if 0 <= int(t) < T})
            else:
                by = global_bits.view(torch.uint8).to(torch.int32)
                n_global = int(((by.unsqueeze(-1) >> torch.arange(8, device=by.device)) & 1)
                               .sum().item())
        need = bwd_window_workspace_bytes(B, H, k.shape[2], T, D, window, n_global, head_split)
        if need < 0:
            raise ValueError("invalid sizes for the backward workspace")
    ptrs, dims, scale, workspace, grads = _bwd_args(q, k, v, o, lse, dout, scale, head_split,
                                                    workspace, need)
    if global_tokens is not None:
        global_bits = window_bitmap(global_tokens, dims[3], q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_bwd_window(*ptrs, *dims, int(bool(causal)), scale, _dtype_code(q),
                              int(window),
                              None if global_bits is None else global_bits.data_ptr(),
                              int(head_split), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), stream)
    _raise(rc, "fa_bwd_window")
    return grads


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale=None, workspace=None,
        head_split: int = 0):
    """Attention backward on contiguous BNHD tensors (bfloat16 or float16).

    q, o, dout: [B, T, H, D]; k, v: [B, T, H_kv, D]; lse: float32 [B, H, T]
    -- o and lse as returned by fwd for the same q, k, v, causal, scale.
    Returns (dq, dk, dv) shaped like q, k, v. `workspace` (optional): a
    device tensor of at least bwd_workspace_bytes(B, H, H_kv, T, D, head_split)
    bytes; allocated here when None. head_split: parts the query heads of a
    kv head are split into for the dK/dV kernel (0: the library's choice)."""
    ptrs, dims, scale, workspace, grads = _bwd_args(q, k, v, o, lse, dout, scale, head_split,
                                                    workspace)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib().fa_bwd(*ptrs, *dims, int(bool(causal)), scale, _dtype_code(q), int(head_split),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       stream)
    _raise(rc, "fa_bwd")
    return grads
