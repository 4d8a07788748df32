"""Pins for the oracle's sliding-window / local-global attention
(oracle.attention_masked): key j is visible to query i iff |i - j| <= window
or j is a global token, and j <= i when causal (yelogs.com Flash
Attention2-in-Triton article, sparse-attention variants).

Each check reaches the same rows another way: a window covering everything
is plain attention; window 0 is each row's own value; all tokens global is
plain attention; and every row equals the merge (pinned lse_combine) of
range-restricted attention (pinned attention_range) over the band and over
each global token outside it -- the visible set built from the predicates
independently of the oracle's own loop.
"""
import numpy as np
import pytest

from exact_attention_91_amd.inputs import generate


def _rand(B, H, H_kv, T, D, seed, sigma=1.0):
    x = generate(B, H, H_kv, T, D, dtype="f32", seed=seed, qk_sigma=sigma)
    return x.q64, x.k64, x.v64


@pytest.mark.parametrize("causal", [False, True])
def test_m1_wide_window_is_plain_attention(oracle, causal):
    q, k, v = _rand(2, 3, 1, 40, 8, seed=1101)
    for w in (39, 40, 1000):
        o, l = oracle.attention_masked(q, k, v, causal, 0.3, w)
        ro, rl = oracle.attention(q, k, v, causal, 0.3)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l, rl, rtol=0, atol=1e-14)


def test_m2_window_zero_is_own_value(oracle):
    """window 0, no global tokens: each row sees only itself."""
    q, k, v = _rand(1, 2, 2, 17, 8, seed=1102)
    for causal in (False, True):
        o, l = oracle.attention_masked(q, k, v, causal, 0.45, 0)
        np.testing.assert_array_equal(o, v)
        s = 0.45 * np.einsum("bthd,bthd->bht", q, k)
        np.testing.assert_allclose(l, s, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_m3_all_global_is_plain_attention(oracle, causal):
    q, k, v = _rand(1, 2, 1, 33, 8, seed=1103)
    o, l = oracle.attention_masked(q, k, v, causal, 0.3, 2, global_tokens=range(33))
    ro, rl = oracle.attention(q, k, v, causal, 0.3)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window,glob", [(3, ()), (5, (0, 1, 20)), (0, (7,)), (12, (2, 39, 40, 63))])
def test_m4_rows_are_merged_ranges(oracle, causal, window, glob):
    """Row i from pinned pieces: attention over the band [i - w, i + w] (cut by
    causality and T) as one key range, each global token outside it as a
    one-key range, merged by their logsumexps."""
    B, H, T, D = 1, 2, 64, 8
    q, k, v = _rand(B, H, 1, T, D, seed=1104 + window)
    o, l = oracle.attention_masked(q, k, v, causal, 0.4, window, global_tokens=glob)
    for i in (0, 1, 5, 31, 40, 63):
        lo = max(0, i - window)
        hi = min(T - 1, i + window, i if causal else T - 1)
        ranges = [(lo, hi + 1)]
        for j in sorted(set(glob)):
            if (j < lo or j > hi) and (not causal or j <= i):
                ranges.append((j, j + 1))
        parts = [oracle.attention_range(q, k, v, False, 0.4, a, b) for a, b in ranges]
        po = np.stack([p_[0][:, :, i] for p_ in parts])     # [n, B, H, D]
        pl = np.stack([p_[1][:, :, i] for p_ in parts])     # [n, B, H]
        ro, rl = oracle.lse_combine(po, pl)
        np.testing.assert_allclose(o[:, i], ro, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[:, :, i], rl, rtol=0, atol=1e-13)


def test_m5_reversal_symmetry(oracle):
    """Non-causal band masks are symmetric: reversing the token order (and
    the global positions) reverses the output rows."""
    B, H, T, D = 1, 2, 50, 8
    q, k, v = _rand(B, H, H, T, D, seed=1105)
    glob = (3, 17, 48)
    o, l = oracle.attention_masked(q, k, v, False, 0.5, 6, global_tokens=glob)
    ro, rl = oracle.attention_masked(q[:, ::-1], k[:, ::-1], v[:, ::-1], False, 0.5, 6,
                                     global_tokens=[T - 1 - j for j in glob])
    np.testing.assert_allclose(o, ro[:, ::-1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, rl[:, :, ::-1], rtol=0, atol=1e-14)


def test_m6_two_visible_keys_closed_form(oracle):
    """Causal, window 0, global token 0: row i > 0 sees keys 0 and i only, so
    O_i = (e^{s_i0} v_0 + e^{s_ii} v_i) / (e^{s_i0} + e^{s_ii})."""
    B, H, T, D = 1, 1, 9, 4
    q, k, v = _rand(B, H, H, T, D, seed=1106)
    o, l = oracle.attention_masked(q, k, v, True, 0.7, 0, global_tokens=(0,))
    for i in range(1, T):
        a = 0.7 * float(q[0, i, 0] @ k[0, 0, 0])
        c = 0.7 * float(q[0, i, 0] @ k[0, i, 0])
        e0, e1 = np.exp(a), np.exp(c)
        np.testing.assert_allclose(o[0, i, 0], (e0 * v[0, 0, 0] + e1 * v[0, i, 0]) / (e0 + e1),
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(l[0, 0, i], np.log(e0 + e1), rtol=0, atol=1e-14)


def test_m7_bad_arguments(oracle):
    q, k, v = _rand(1, 1, 1, 8, 4, seed=1107)
    with pytest.raises(ValueError):
        oracle.attention_masked(q, k, v, False, 1.0, 2, global_tokens=(8,))
    with pytest.raises(RuntimeError):
        oracle.attention_masked(q, k, v, False, 1.0, -1)


# ------------------------------------------------- gradients under the masks

def _rand_do(q, seed):
    return np.random.default_rng(seed).standard_normal(q.shape)


@pytest.mark.parametrize("causal", [False, True])
def test_mb1_wide_window_is_plain_backward(oracle, causal):
    q, k, v = _rand(2, 4, 2, 37, 8, seed=1201)
    do = _rand_do(q, 1202)
    a = oracle.attention_bwd_masked(q, k, v, do, causal, 0.3, 36)
    b = oracle.attention_bwd(q, k, v, do, causal, 0.3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window,glob", [(1, ()), (2, (0, 6)), (0, (3,))])
def test_mb2_finite_differences(oracle, causal, window, glob):
    """Central differences of loss = sum(O * dO) through the pinned masked
    forward."""
    B, H, T, D = 1, 2, 7, 3
    q, k, v = _rand(B, H, 1, T, D, seed=1203 + window)
    do = _rand_do(q, 1204)
    scale = 0.8
    grads = oracle.attention_bwd_masked(q, k, v, do, causal, scale, window, glob)

    def loss(q, k, v):
        o, _ = oracle.attention_masked(q, k, v, causal, scale, window, glob)
        return float(np.sum(o * do))

    h = 1e-5
    for name, g in zip(("q", "k", "v"), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = args[name].copy(), args[name].copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (loss(**dict(args, **{name: xp})) -
                        loss(**dict(args, **{name: xm}))) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_mb3_torch_autograd_with_explicit_mask(oracle, causal):
    """torch float64 autograd through the naive module with the mask built
    from the pages' predicates (|i - j| <= w or isin(j, globals), and j <= i
    when causal) as a masked_fill of -inf."""
    import torch
    B, H, H_kv, T, D = 2, 4, 2, 41, 16
    window, glob = 5, (0, 20, 40)
    q, k, v = _rand(B, H, H_kv, T, D, seed=1205, sigma=1.5)
    do = _rand_do(q, 1206)
    scale = 0.25
    dq, dk, dv = oracle.attention_bwd_masked(q, k, v, do, causal, scale, window, glob)
    g = H // H_kv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    qh = tq.permute(0, 2, 1, 3)
    kh = tk.permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vh = tv.permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    s = scale * torch.matmul(qh, kh.transpose(-1, -2).contiguous())
    qi = torch.arange(T)[:, None]
    kj = torch.arange(T)[None, :]
    visible = (torch.abs(qi - kj) <= window) | torch.isin(kj, torch.tensor(glob))
    if causal:
        visible = visible & (kj <= qi)
    p = torch.softmax(s.masked_fill(~visible, float("-inf")), dim=-1)
    o = torch.matmul(p, vh).permute(0, 2, 1, 3)
    o.backward(torch.tensor(do))
    for name, a, b in (("dq", dq, tq.grad.numpy()), ("dk", dk, tk.grad.numpy()),
                       ("dv", dv, tv.grad.numpy())):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_mb4_invariants(oracle, causal):
    """Each row's softmax over its visible keys is shift invariant and sums to
    1: dK of a kv head sums to zero, dV sums to the group's dO."""
    B, H, H_kv, T, D = 1, 4, 2, 50, 8
    q, k, v = _rand(B, H, H_kv, T, D, seed=1207)
    do = _rand_do(q, 1208)
    dq, dk, dv = oracle.attention_bwd_masked(q, k, v, do, causal, 0.4, 4, (0, 25))
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
    do_groups = do.reshape(B, T, H_kv, H // H_kv, D).sum(axis=3).sum(axis=1)
    np.testing.assert_allclose(dv.sum(axis=1), do_groups, rtol=0, atol=1e-12)
