"""The score range the 16-bit and fp32 forward kernels support (include/fa.h,
"Range"), checked on the CPU by emulating their per-row weight arithmetic in
IEEE float32.

The kernels form the weights as exp2(fma(s, c, -m)): s the fp32 raw score
(q.k), c = |scale| * log2(e) in fp32, m = fp32(max_j s_j * c) the rounded
running max. fma rounds once, after the exact s*c - m, so every weight of a row
carries the same factor 2^(max s*c - m); it cancels in O = sum P v / sum P and
in L = (m + log2 sum P) ln 2, as long as exp2 of it stays finite: |max s*c -
m| <= ulp(m) / 2 <= 64 whenever |s*c| < 2^31. These tests pin that bound (and
show it is needed) with exact float64 references; no GPU is involved.
"""
import numpy as np
import pytest

LOG2E = 1.4426950408889634
BOUND = 2.0 ** 31 / LOG2E          # |scale * q.k| below this is supported (~1.49e9)


def emulated_row(s, scale):
    """Weights, O-normalised weights and L of one row as the kernels compute
    them: s float32 scores, fp32 c and m, weights exp2 of the fma result (the
    fma emulated exactly in float64: a product of two float32 values is exact
    in float64, and so is its difference with a float32 of similar size)."""
    s = np.asarray(s, dtype=np.float32)
    c = np.float32(abs(scale) * LOG2E)
    m = np.float32(np.max(s) * c)                       # v_mul_f32, rounded
    t = (s.astype(np.float64) * np.float64(c) - np.float64(m)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        p = np.exp2(t.astype(np.float64)).astype(np.float32)
        l = np.float32(np.sum(p, dtype=np.float64))
        L = (np.float64(m) + np.log2(np.float64(l))) * np.log(2.0)
        return p, p / l, L


def reference_row(s, scale):
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64) * (abs(scale) * LOG2E)
    w = np.exp2(s64 - s64.max())
    return w / w.sum(), (s64.max() + np.log2(w.sum())) * np.log(2.0)


@pytest.mark.parametrize("mag", [1e3, 1e6, 1e9, 1.45e9, -1e9, -1.45e9])
def test_weights_finite_and_exact_within_bound(mag):
    """Rows of scores up to the documented bound: the shared factor stays
    within 2^-64..2^64, and the normalised weights and L match float64."""
    rng = np.random.default_rng(11)
    scale = 0.125
    assert abs(mag) < BOUND
    for _ in range(200):
        # scores near the magnitude, spread over a few units (so rows are not
        # one-hot) and over many ulps of the magnitude
        raw = np.float32(mag / scale) + rng.uniform(-8, 8, size=64).astype(np.float32) * \
            np.float32(max(1.0, abs(mag) * 2.0 ** -20) / scale)
        p, pn, L = emulated_row(raw, scale)
        assert np.all(np.isfinite(p)) and np.max(p) >= 2.0 ** -64 and np.max(p) <= 2.0 ** 64
        ref_pn, ref_L = reference_row(raw, scale)
        assert np.max(np.abs(pn - ref_pn)) < 1e-5
        assert abs(L - ref_L) <= 1e-3 + 1e-6 * abs(ref_L)


def test_bound_is_needed():
    """Beyond the bound the shared factor can leave fp32 range: at |s*c| near
    2^40 the rounding error of m reaches 2^16, and exp2 of it overflows."""
    scale = 1.0
    found = False
    rng = np.random.default_rng(12)
    for _ in range(2000):
        x = np.float32(2.0 ** 40 / LOG2E * rng.uniform(1.0, 1.9))
        p, _, _ = emulated_row(np.array([x], dtype=np.float32), scale)
        if not np.isfinite(p[0]) or p[0] == 0.0:
            found = True
            break
    assert found


def test_documented_bound_in_header():
    """fa.h states the same bound."""
    import os
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "include", "fa.h")).read()
    assert "|scale * q.k| < 1.4e9" in text and "2^31" in text
    assert 1.4e9 < BOUND < 1.5e9
