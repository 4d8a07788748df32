"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare with the float64 oracle."""
import sys

import numpy as np
import torch

# Tolerances on max |GPU - oracle|: fp32 in/out 1e-4 on O and L; bf16 in with
# fp32 accumulation 2e-2 on O and 1e-3 on L. fp16: 5e-3 on O, 1e-3 on L --
# the weights are rounded to half (relative 2^-11) for P.V and O to half
# (half an ulp is <= 2^-9 for |O| < 8), so |dO| stays below ~2^-9 + 8*2^-11
# ~ 6e-3 in the worst case of a one-hot row with |v| ~ 4; L is computed in fp32.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3), "f16": (5e-3, 1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(x):
    return x.q.cuda(), x.k.cuda(), x.v.cuda()


def run_gpu(x, causal, scale):
    from exact_attention_91_amd import fa
    q, k, v = to_gpu(x)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def max_err(a, b):
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def check_full(x, dtype, causal, scale, o_gpu, l_gpu, label=""):
    from oracle import oracle as orc
    o_ref, l_ref = orc.attention(x.q64, x.k64, x.v64, causal, scale)
    eo, el = max_err(o_gpu, o_ref), max_err(l_gpu, l_ref)
    tol_o, tol_l = TOL[dtype]
    say(f"  {label} max|dO|={eo:.3e} (tol {tol_o}) max|dL|={el:.3e} (tol {tol_l})")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(l_gpu))
    assert eo <= tol_o, f"O error {eo} > {tol_o}"
    assert el <= tol_l, f"L error {el} > {tol_l}"
    return eo, el


def check_rows(x, dtype, causal, scale, o_gpu, l_gpu, rows, label=""):
    from oracle import oracle as orc
    B, T, H, D = x.q64.shape
    o_ref, l_ref = orc.attention_rows(x.q64, x.k64, x.v64, causal, scale, rows)
    b, rem = rows // (H * T), rows % (H * T)
    h, i = rem // T, rem % T
    og = o_gpu[b, i, h]
    lg = l_gpu[b, h, i]
    eo, el = max_err(og, o_ref), max_err(lg, l_ref)
    tol_o, tol_l = TOL[dtype]
    say(f"  {label} rows={len(rows)} max|dO|={eo:.3e} (tol {tol_o}) "
        f"max|dL|={el:.3e} (tol {tol_l})")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(l_gpu))
    assert eo <= tol_o, f"O error {eo} > {tol_o}"
    assert el <= tol_l, f"L error {el} > {tol_l}"
    return eo, el
