"""Pins for the oracle's decode-shaped attention (oracle_attn_decode_f64):
T_q query rows, the last T_q positions of a T_k-long sequence, against T_k
keys; under the causal mask query i sees keys j <= T_k - T_q + i.

Each test checks it against something other than itself: the square oracle
(itself pinned) on the rows the decode rows must equal, a pure-Python brute
force with hand-expanded exponentials and no max subtraction, and closed forms
(zero queries average the visible values; rows with no visible key).
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_square_oracle(causal):
    B, T, H, H_kv, D = 2, 37, 4, 2, 16
    q, k, v = _rand((B, T, H, D), 1), _rand((B, T, H_kv, D), 2), _rand((B, T, H_kv, D), 3)
    o1, l1 = orc.attention_decode(q, k, v, causal, 0.3)
    o2, l2 = orc.attention(q, k, v, causal, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(1, 50), (3, 50), (8, 9), (16, 100)])
def test_rows_are_the_last_rows_of_square_attention(causal, Tq, Tk):
    """The decode rows are the last T_q rows of attention over the full
    T_k-long sequence (whatever its earlier query rows hold): this pins the
    position offset of the causal mask."""
    B, H, H_kv, D = 2, 6, 3, 8
    q = _rand((B, Tq, H, D), 4)
    k, v = _rand((B, Tk, H_kv, D), 5), _rand((B, Tk, H_kv, D), 6)
    qfull = _rand((B, Tk, H, D), 7)
    qfull[:, Tk - Tq:] = q
    o_full, l_full = orc.attention(qfull, k, v, causal, 0.25)
    o, l = orc.attention_decode(q, k, v, causal, 0.25)
    assert np.max(np.abs(o - o_full[:, Tk - Tq:])) < 1e-13
    assert np.max(np.abs(l - l_full[:, :, Tk - Tq:])) < 1e-13


def _brute(q, k, v, causal, scale):
    B, Tq, H, D = q.shape
    Tk, H_kv = k.shape[1], k.shape[2]
    o = np.zeros((B, Tq, H, D))
    lse = np.zeros((B, H, Tq))
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            for i in range(Tq):
                keys = [j for j in range(Tk) if not causal or j <= Tk - Tq + i]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                e = [(j, math.exp(scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d])
                                                     for d in range(D)))) for j in keys]
                z = math.fsum(w for _, w in e)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(w * float(v[b, j, g, d]) for j, w in e) / z
                lse[b, h, i] = math.log(z)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 7), (2, 5), (4, 8), (6, 3)])
def test_brute_force_small(causal, Tq, Tk):
    B, H, H_kv, D = 1, 4, 2, 5
    q = _rand((B, Tq, H, D), 8)
    k, v = _rand((B, Tk, H_kv, D), 9), _rand((B, Tk, H_kv, D), 10)
    o, l = orc.attention_decode(q, k, v, causal, 0.7)
    ob, lb = _brute(q, k, v, causal, 0.7)
    assert np.max(np.abs(o - ob)) < 1e-12
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.max(np.abs(l[fin] - lb[fin])) < 1e-12


def test_zero_queries_average_the_visible_values():
    """q = 0: every visible key has weight 1/n, so O is the mean of the first
    n values and L = ln n, with n = T_k - T_q + i + 1 under the causal mask;
    rows before the cache (T_q > T_k) see nothing: O = 0, L = -inf."""
    B, Tq, Tk, H, H_kv, D = 2, 7, 5, 2, 1, 4
    q = np.zeros((B, Tq, H, D))
    k, v = _rand((B, Tk, H_kv, D), 11), _rand((B, Tk, H_kv, D), 12)
    o, l = orc.attention_decode(q, k, v, True, 0.5)
    for i in range(Tq):
        n = Tk - Tq + i + 1
        if n <= 0:
            assert np.all(o[:, i] == 0.0) and np.all(l[:, :, i] == -np.inf)
        else:
            mean = v[:, :n, 0, :].mean(axis=1)
            for h in range(H):
                assert np.max(np.abs(o[:, i, h] - mean)) < 1e-14
            assert np.max(np.abs(l[:, :, i] - math.log(n))) < 1e-14
    o, l = orc.attention_decode(q, k, v, False, 0.5)
    assert np.max(np.abs(o[:, :, 0] - v[:, :, 0].mean(axis=1)[:, None])) < 1e-14


def test_bad_shapes_rejected():
    q = np.zeros((1, 2, 4, 8))
    with pytest.raises(ValueError):
        orc.attention_decode(q, np.zeros((1, 5, 3, 8)), np.zeros((1, 5, 3, 8)), True, 1.0)
    with pytest.raises(ValueError):
        orc.attention_decode(q, np.zeros((1, 5, 2, 4)), np.zeros((1, 5, 2, 4)), True, 1.0)
