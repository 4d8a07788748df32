"""Tensors past 2^31 elements (4.6 GB): the kernels' 64-bit offsets.

q and o of [136, 8192, 16, 128] bf16 hold 2.28e9 elements each, past what a
signed 32-bit index (elements) or an unsigned one (bytes) can address; one kv
head keeps k and v at 285 MB. The inputs are drawn on the device by torch's seeded generator
(plain N(0, 1) in fp32, rounded to bf16), so nothing this size is built on the
host. Sampled rows -- the first and last batch, head and token among them, so
the largest offsets are read and written -- are compared with the oracle run
on each row's own problem: that row's query at its position i against the
keys of its batch it sees (0..i when causal, all T otherwise).
Tolerances as every bf16 parity test: 2e-2 on O, 1e-3 on L.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _randn_bf16(shape, g):
    return torch.randn(shape, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_tensors_past_2e31_elements(causal):
    from exact_attention_91_amd import fa
    from oracle import oracle as orc
    B, T, H, H_kv, D = 136, 8192, 16, 1, 128
    assert B * T * H * D > 2 ** 31 and B * T * H * D * 2 > 2 ** 32
    g = torch.Generator(device="cuda")
    g.manual_seed(31337 + int(causal))
    q = _randn_bf16((B, T, H, D), g)
    k = _randn_bf16((B, T, H_kv, D), g)
    v = _randn_bf16((B, T, H_kv, D), g)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    say(f"case large fwd causal={causal} B={B} T={T} H={H} H_kv={H_kv} D={D}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4711)
    rows = [(0, 0, 0), (B - 1, H - 1, T - 1), (B - 1, 0, T - 1), (0, H - 1, T - 1),
            (B - 1, H - 1, 0), (B // 2, 7, 4095)]
    rows += [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T)))
             for _ in range(10)]
    tol_o, tol_l = TOL["bf16"]
    for b, h, i in rows:
        n = i + 1 if causal else T
        # the row's own problem: its batch's first n keys (all it sees) and its
        # query at position i (the other queries are zero and not evaluated)
        q1 = np.zeros((1, n, 1, D))
        q1[0, i, 0] = q[b, i, h].to(torch.float64).cpu().numpy()
        k1 = k[b, :n, 0].to(torch.float64).cpu().numpy().reshape(1, n, 1, D)
        v1 = v[b, :n, 0].to(torch.float64).cpu().numpy().reshape(1, n, 1, D)
        ro, rl = orc.attention_rows(q1, k1, v1, causal, scale, [i])
        go = o[b, i, h].to(torch.float64).cpu().numpy()
        gl = float(lse[b, h, i])
        eo = float(np.max(np.abs(go - ro[0])))
        el = abs(gl - float(rl[0]))
        say(f"  row b={b} h={h} i={i}: |dO|={eo:.2e} |dL|={el:.2e}")
        assert eo <= tol_o and el <= tol_l, (b, h, i, eo, el)
    b = B - 1
    o1, l1 = fa.fwd(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                    causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o[b:b + 1], o1) and torch.equal(lse[b:b + 1], l1)
    say("  last batch alone: bitwise equal")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_bwd_tensors_past_2e31_elements():
    """Backward with q, o, dO and dQ of 4.6 GB each (head split 1). dQ of sampled
    rows from each row's own problem (its query and dO at position i; row i's
    gradient depends on no other query row), to 2e-2 x
    max(1, max|ref|) as every bf16 backward test. The first, a middle and the
    last batch are then run again within nine-batch slices (small offsets; nine
    batches keep more than 512 key-tile work-groups, so the library picks the
    same dK/dV kernel as for the large run): each work-group computes the same
    values in the same order, so o, lse, dQ, dK and dV of those batches must be
    bitwise those of the large run."""
    from exact_attention_91_amd import fa
    from oracle import oracle as orc
    B, T, H, H_kv, D = 136, 8192, 16, 1, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    q = _randn_bf16((B, T, H, D), g)
    k = _randn_bf16((B, T, H_kv, D), g)
    v = _randn_bf16((B, T, H_kv, D), g)
    do = _randn_bf16((B, T, H, D), g)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    say(f"case large bwd B={B} T={T} H={H} H_kv={H_kv} D={D}")
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, head_split=1)
    torch.cuda.synchronize()

    def f64(t):
        return t.to(torch.float64).cpu().numpy()

    rtol = 2e-2
    rng = np.random.default_rng(4713)
    rows = [(B - 1, H - 1, T - 1), (B - 1, 0, T - 1), (0, 0, 0), (B - 1, H - 1, 4000)]
    rows += [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T)))
             for _ in range(6)]
    for b, h, i in rows:
        n = i + 1
        q1 = np.zeros((1, n, 1, D))
        d1 = np.zeros((1, n, 1, D))
        q1[0, i, 0] = f64(q[b, i, h])
        d1[0, i, 0] = f64(do[b, i, h])
        ref = orc.attention_bwd_dq_rows(q1, f64(k[b:b + 1, :n]), f64(v[b:b + 1, :n]), d1, True,
                                        scale, [i])[0]
        err = float(np.max(np.abs(f64(dq[b, i, h]) - ref)))
        tol = rtol * max(1.0, float(np.max(np.abs(ref))))
        say(f"  dq row b={b} h={h} i={i}: |err|={err:.2e} (tol {tol:.2e})")
        assert err <= tol, (b, h, i, err)
    nsl = 9
    for b in (0, B // 2, B - 1):
        b0 = min(b, B - nsl)
        j = b - b0
        sl = [t[b0:b0 + nsl].contiguous() for t in (q, k, v, do)]
        o1, l1 = fa.fwd(sl[0], sl[1], sl[2], causal=True, scale=scale)
        g1 = fa.bwd(sl[0], sl[1], sl[2], o1, l1, sl[3], causal=True, scale=scale, head_split=1)
        torch.cuda.synchronize()
        for name, big, small in (("o", o[b], o1[j]), ("lse", lse[b], l1[j]),
                                 ("dq", dq[b], g1[0][j]), ("dk", dk[b], g1[1][j]),
                                 ("dv", dv[b], g1[2][j])):
            assert torch.equal(big, small), (b, name)
        say(f"  batch {b} in a {nsl}-batch slice: o, lse, dq, dk, dv bitwise equal")
        del sl, o1, l1, g1
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_window_tensors_past_2e31_elements():
    """Window forward and backward (window 64, causal, global tokens, far split)
    on [272, 8192, 16, 64] q: the last batch run alone is bitwise the large
    run's, and that batch is compared in full with the masked oracle (O to
    2e-2, L to 1e-3; gradients to 2e-2 x max(1, max|ref|))."""
    from exact_attention_91_amd import fa
    from oracle import oracle as orc
    B, T, H, H_kv, D = 272, 8192, 16, 1, 64
    assert B * T * H * D > 2 ** 31
    window, glob = 64, (0, 1, 4000, 8191)
    g = torch.Generator(device="cuda")
    g.manual_seed(4343)
    q = _randn_bf16((B, T, H, D), g)
    k = _randn_bf16((B, T, H_kv, D), g)
    v = _randn_bf16((B, T, H_kv, D), g)
    do = _randn_bf16((B, T, H, D), g)
    scale = 0.125
    say(f"case large window B={B} T={T} H={H} D={D} window={window} globals={glob}")
    bits = fa.window_bitmap(glob, T, q.device)

    def run(q_, k_, v_, do_):
        b_ = q_.shape[0]
        o_, l_ = fa.fwd_window(q_, k_, v_, window, causal=True, scale=scale, global_bits=bits)
        ws = torch.empty((fa.bwd_window_workspace_bytes(b_, H, H_kv, T, D, window, len(glob),
                                                        1),), dtype=torch.uint8, device="cuda")
        g_ = fa.bwd_window(q_, k_, v_, o_, l_, do_, window, causal=True, scale=scale,
                           global_bits=bits, head_split=1, workspace=ws)
        return (o_, l_) + tuple(g_)

    big = run(q, k, v, do)
    torch.cuda.synchronize()
    b = B - 1
    small = run(*(t[b:b + 1].contiguous() for t in (q, k, v, do)))
    torch.cuda.synchronize()
    for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), big, small):
        assert torch.equal(x[b:b + 1], y), name
    say("  last batch alone: bitwise equal")

    def f64(t):
        return t.to(torch.float64).cpu().numpy()

    q1, k1, v1, d1 = (f64(t[b:b + 1]) for t in (q, k, v, do))
    ro, rl = orc.attention_masked(q1, k1, v1, True, scale, window, glob)
    eo, el = float(np.max(np.abs(f64(small[0]) - ro))), float(np.max(np.abs(f64(small[1]) - rl)))
    say(f"  oracle: |dO|={eo:.2e} |dL|={el:.2e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]
    ref = orc.attention_bwd_masked(q1, k1, v1, d1, True, scale, window, glob)
    for name, got, r in zip(("dq", "dk", "dv"), small[2:], ref):
        err = float(np.max(np.abs(f64(got) - r)))
        tol = 2e-2 * max(1.0, float(np.max(np.abs(r))))
        say(f"  oracle {name}: |err|={err:.2e} (tol {tol:.2e})")
        assert err <= tol, (name, err, tol)
    del q, k, v, do, big, small
    torch.cuda.empty_cache()
