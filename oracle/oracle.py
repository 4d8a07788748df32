"""float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU product path never does and shares
no code with it.

Layout everywhere: q, o are [B, T, H, D]; k, v are [B, T, H_kv, D]; lse is
[B, H, T]. Query head h reads kv head h // (H // H_kv).

Functions
---------
attention(q, k, v, causal, scale)        two-pass softmax over the whole row
                                         (C, OpenMP), the plain definition.
attention_rows(..., rows)                the same for selected flat rows
attention_bwd_dq_rows(..., rows)         dQ of selected flat rows (backward)
                                         (b*H + h)*T + i.
attention_online(..., chunk)             the online-softmax recurrence over key
                                         chunks (C), used to show it reaches the
                                         two-pass result.
attention_range(..., lo, hi)             attention over keys [lo, hi) only,
                                         normalised over them (C); partial
                                         results for a key split.
lse_combine(o_parts, lse_parts)          merge of partials over disjoint key
                                         ranges: L = ln sum exp(L_s),
                                         O = sum exp(L_s - L) O_s (C).
attention_masked(q, k, v, causal, scale, window, global_tokens)
                                         sliding-window / local-global mask:
                                         key j visible to query i iff
                                         |i - j| <= window or j is a global
                                         token (and j <= i when causal) (C).
attention_bwd(q, k, v, dout, causal, scale)
                                         gradients (dq, dk, dv) of the same
                                         definition for upstream gradient dO,
                                         every intermediate recomputed (C).
attention_bwd_masked(q, k, v, dout, causal, scale, window, global_tokens)
                                         gradients of attention_masked (C).
brute_force(q, k, v, causal, scale)      pure Python, hand-expanded exponentials
                                         summed with math.fsum, no max
                                         subtraction; for T <= 8 only.

Sources: the yelogs.com Flash Attention2-in-Triton article, sections
"問題的根源：傳統注意力機制的痛點" (naive module), "核心思想：分塊計算與在線更新"
(traditional and online softmax), "因果掩碼的高效實現" (causal predicate: query
position >= key position), "Softmax 的在線計算" (recurrence), "核心 Kernel 實現"
(stored statistic m + ln l), "多查詢注意力（MQA）" (shared kv head); and
"Flash Attention Memory Optimization Explained", "What is Flash Attention?"
(the four naive steps), "Key Mechanisms" (backward checkpointing: the backward
pass recomputes intermediates instead of storing them; its formulas are the
chain rule of the naive steps).
"""
import ctypes
import math
import os

import numpy as np

from . import build_oracle

_LIB = None
_DP = ctypes.POINTER(ctypes.c_double)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(build_oracle.LIB):
            build_oracle.build()
        lib = ctypes.CDLL(build_oracle.LIB)
        common = [_DP, _DP, _DP]
        shape = [ctypes.c_int] * 5 + [ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_f64.argtypes = common + [_DP, _DP] + shape
        lib.oracle_attn_f64.restype = ctypes.c_int
        lib.oracle_attn_rows_f64.argtypes = (
            common + [ctypes.POINTER(ctypes.c_int64), ctypes.c_longlong, _DP, _DP] + shape)
        lib.oracle_attn_rows_f64.restype = ctypes.c_int
        lib.oracle_attn_online_f64.argtypes = common + [_DP, _DP] + shape + [ctypes.c_int]
        lib.oracle_attn_online_f64.restype = ctypes.c_int
        lib.oracle_attn_range_f64.argtypes = (common + [_DP, _DP] + shape +
                                              [ctypes.c_int, ctypes.c_int])
        lib.oracle_attn_range_f64.restype = ctypes.c_int
        lib.oracle_lse_combine_f64.argtypes = [_DP, _DP, ctypes.c_int, ctypes.c_longlong,
                                               ctypes.c_int, _DP, _DP]
        lib.oracle_lse_combine_f64.restype = ctypes.c_int
        lib.oracle_attn_masked_f64.argtypes = (common + [_DP, _DP] + shape +
                                               [ctypes.c_int, ctypes.c_void_p])
        lib.oracle_attn_masked_f64.restype = ctypes.c_int
        lib.oracle_attn_bwd_f64.argtypes = common + [_DP, _DP, _DP, _DP] + shape
        lib.oracle_attn_bwd_f64.restype = ctypes.c_int
        lib.oracle_attn_bwd_masked_f64.argtypes = (common + [_DP, _DP, _DP, _DP] + shape +
                                                   [ctypes.c_int, ctypes.c_void_p])
        lib.oracle_attn_bwd_masked_f64.restype = ctypes.c_int
        lib.oracle_attn_bwd_dq_rows_f64.argtypes = (
            [_DP, _DP, _DP, _DP, ctypes.POINTER(ctypes.c_int64), ctypes.c_longlong, _DP] +
            [ctypes.c_int] * 5 + [ctypes.c_int, ctypes.c_double])
        lib.oracle_attn_bwd_dq_rows_f64.restype = ctypes.c_int
        lib.oracle_attn_decode_f64.argtypes = (common + [_DP, _DP] + [ctypes.c_int] * 6 +
                                               [ctypes.c_int, ctypes.c_double])
        lib.oracle_attn_decode_f64.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        _LIB = lib
    return _LIB


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_DP)


def _shape(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, T, heads, D]")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError(f"k/v shape {k.shape} does not match q {q.shape}")
    H_kv = k.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return B, H, H_kv, T, D


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle uses from now on (OpenMP)."""
    _lib().oracle_set_num_threads(int(n))


def attention(q, k, v, causal: bool, scale: float):
    """Two-pass float64 attention. Returns (o [B,T,H,D], lse [B,H,T])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, H_kv, T, D = _shape(q, k, v)
    o = np.empty((B, T, H, D), np.float64)
    lse = np.empty((B, H, T), np.float64)
    rc = _lib().oracle_attn_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                B, H, H_kv, T, D, int(bool(causal)), float(scale))
    if rc:
        raise RuntimeError(f"oracle_attn_f64 failed ({rc})")
    return o, lse


def attention_decode(q, k, v, causal: bool, scale: float):
    """T_q query rows (the last T_q positions) against T_k keys: q [B, T_q, H, D],
    k, v [B, T_k, H_kv, D]. Returns (o [B, T_q, H, D], lse [B, H, T_q])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
        raise ValueError("q [B, T_q, H, D] and k, v [B, T_k, H_kv, D] expected")
    B, Tq, H, D = q.shape
    Tk, H_kv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or H % H_kv:
        raise ValueError(f"k/v shape {k.shape} does not match q {q.shape}")
    o = np.empty((B, Tq, H, D), np.float64)
    lse = np.empty((B, H, Tq), np.float64)
    rc = _lib().oracle_attn_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       B, H, H_kv, Tq, Tk, D, int(bool(causal)), float(scale))
    if rc:
        raise RuntimeError(f"oracle_attn_decode_f64 failed ({rc})")
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, rows):
    """Rows given as flat ids (b*H + h)*T + i. Returns (o [n, D], lse [n])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, H_kv, T, D = _shape(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _lib().oracle_attn_rows_f64(
        _ptr(q), _ptr(k), _ptr(v), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        n, _ptr(o), _ptr(lse), B, H, H_kv, T, D, int(bool(causal)), float(scale))
    if rc:
        raise RuntimeError(f"oracle_attn_rows_f64 failed ({rc})")
    return o, lse


def attention_bwd_dq_rows(q, k, v, dout, causal: bool, scale: float, rows):
    """dQ of selected rows (flat ids (b*H + h)*T + i), plain or causal mask.
    Returns dq [n, D]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, H_kv, T, D = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    dq = np.empty((n, D), np.float64)
    rc = _lib().oracle_attn_bwd_dq_rows_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, _ptr(dq),
        B, H, H_kv, T, D, int(bool(causal)), float(scale))
    if rc:
        raise RuntimeError(f"oracle_attn_bwd_dq_rows_f64 failed ({rc})")
    return dq


def attention_online(q, k, v, causal: bool, scale: float, chunk: int):
    """Online-softmax recurrence over key chunks. Returns (o, lse)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, H_kv, T, D = _shape(q, k, v)
    o = np.empty((B, T, H, D), np.float64)
    lse = np.empty((B, H, T), np.float64)
    rc = _lib().oracle_attn_online_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       B, H, H_kv, T, D, int(bool(causal)), float(scale),
                                       int(chunk))
    if rc:
        raise RuntimeError(f"oracle_attn_online_f64 failed ({rc})")
    return o, lse


def attention_range(q, k, v, causal: bool, scale: float, lo: int, hi: int):
    """Attention over keys [lo, hi) only (intersected with the visible set),
    normalised over those keys. Returns (o_part [B, H, T, D], lse_part
    [B, H, T]); an empty range gives o_part = 0 and lse_part = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, H_kv, T, D = _shape(q, k, v)
    o = np.empty((B, H, T, D), np.float64)
    lse = np.empty((B, H, T), np.float64)
    rc = _lib().oracle_attn_range_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      B, H, H_kv, T, D, int(bool(causal)), float(scale),
                                      int(lo), int(hi))
    if rc:
        raise RuntimeError(f"oracle_attn_range_f64 failed ({rc})")
    return o, lse


def lse_combine(o_parts, lse_parts):
    """Merge partials over disjoint key ranges. o_parts [n, ..., D] and
    lse_parts [n, ...] (any common row shape). Returns (o [..., D], lse [...])."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    n = o_parts.shape[0]
    D = o_parts.shape[-1]
    row_shape = lse_parts.shape[1:]
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing D")
    rows = int(np.prod(row_shape)) if row_shape else 1
    o = np.empty(row_shape + (D,), np.float64)
    lse = np.empty(row_shape, np.float64)
    rc = _lib().oracle_lse_combine_f64(_ptr(o_parts), _ptr(lse_parts), n, rows, D,
                                       _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError(f"oracle_lse_combine_f64 failed ({rc})")
    return o, lse


def attention_masked(q, k, v, causal: bool, scale: float, window: int, global_tokens=()):
    """Attention where key j is visible to query i iff |i - j| <= window or j
    is in global_tokens (yelogs.com Flash Attention2-in-Triton article,
    sparse-attention variants: sliding_window_mask, local_global_mask), and
    j <= i when causal. Returns (o, lse) like attention()."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, H_kv, T, D = _shape(q, k, v)
    flags = np.zeros(T, np.uint8)
    for j in global_tokens:
        if not 0 <= int(j) < T:
            raise ValueError(f"global token {j} outside [0, {T})")
        flags[int(j)] = 1
    o = np.empty_like(q)
    lse = np.empty((B, H, T), np.float64)
    rc = _lib().oracle_attn_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                       H_kv, T, D, int(bool(causal)), float(scale), int(window),
                                       flags.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_attn_masked_f64 failed ({rc})")
    return o, lse


def attention_bwd(q, k, v, dout, causal: bool, scale: float):
    """Gradients of attention for upstream gradient dout (same shape as q).
    Returns (dq [B, T, H, D], dk, dv [B, T, H_kv, D]); dk and dv of a shared
    kv head are summed over its query heads."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, H_kv, T, D = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _lib().oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, H_kv, T, D, int(bool(causal)), float(scale))
    if rc:
        raise RuntimeError(f"oracle_attn_bwd_f64 failed ({rc})")
    return dq, dk, dv


def attention_bwd_masked(q, k, v, dout, causal: bool, scale: float, window: int,
                         global_tokens=()):
    """Gradients of attention_masked (same visible sets) for upstream gradient
    dout. Returns (dq, dk, dv) like attention_bwd."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, H_kv, T, D = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    flags = np.zeros(T, np.uint8)
    for j in global_tokens:
        if not 0 <= int(j) < T:
            raise ValueError(f"global token {j} outside [0, {T})")
        flags[int(j)] = 1
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    rc = _lib().oracle_attn_bwd_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                           _ptr(dk), _ptr(dv), B, H, H_kv, T, D,
                                           int(bool(causal)), float(scale), int(window),
                                           flags.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_attn_bwd_masked_f64 failed ({rc})")
    return dq, dk, dv


def brute_force(q, k, v, causal: bool, scale: float):
    """Pure-Python attention for tiny inputs (T <= 8).

    Every weight is written out as exp(score) / fsum(exp(scores)), with no max
    subtraction, and L = ln(fsum(exp(scores))). Scores must stay moderate
    (|score| < 700) for this to be valid.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, H_kv, T, D = _shape(q, k, v)
    if T > 8:
        raise ValueError("brute_force is for T <= 8")
    o = np.zeros((B, T, H, D), np.float64)
    lse = np.zeros((B, H, T), np.float64)
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            for i in range(T):
                keys = [j for j in range(T) if (not causal) or j <= i]
                e = []
                for j in range(T):
                    if j not in keys:
                        continue
                    sc = scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d])
                                           for d in range(D))
                    e.append((j, math.exp(sc)))
                z = math.fsum(w for _, w in e)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(w * float(v[b, j, g, d]) for j, w in e) / z
                lse[b, h, i] = math.log(z)
    return o, lse
