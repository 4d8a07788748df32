"""Sliding-window / local-global forward (fa_fwd_window) through the C ABI
against the float64 oracle (oracle.attention_masked): key j visible to query
i iff |i - j| <= window or j is a global token, and j <= i when causal.
Same tolerances as the plain forward."""
import numpy as np
import pytest
import torch

from exact_attention_91_amd.inputs import WORKLOADS, default_scale, generate, generate_workload
from tests.gpu_util import TOL, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_window(x, causal, scale, window, glob):
    from exact_attention_91_amd import fa
    o, lse = fa.fwd_window(x.q.cuda(), x.k.cuda(), x.v.cuda(), window, glob, causal=causal,
                           scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(x, dtype, causal, scale, window, glob, o, lse, label=""):
    from oracle import oracle as orc
    valid = [int(g) for g in glob if 0 <= int(g) < x.q64.shape[1]]
    ro, rl = orc.attention_masked(x.q64, x.k64, x.v64, causal, scale, window, valid)
    eo, el = max_err(o, ro), max_err(lse, rl)
    say(f"  {label} max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert eo <= TOL[dtype][0] and el <= TOL[dtype][1], (eo, el)


CASES = [  # T, window, global tokens
    (1, 0, ()),
    (65, 0, ()),
    (65, 3, (0,)),
    (300, 1, ()),
    (300, 63, (0, 64, 299)),
    (300, 64, ()),
    (1000, 100, (0, 1, 2, 3)),
    (1000, 257, (5, 500, 999)),
    (1000, 2000, ()),
    (777, 31, tuple(range(0, 777, 97))),
    (1000, 20, tuple(range(1, 1000, 3))),      # 333 tokens: the list is staged in chunks
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,window,glob", CASES)
def test_window_small_elementwise(dtype, D, causal, T, window, glob):
    B, H, H_kv = (2, 3, 1) if T < 500 else (1, 2, 2)
    seed = 9800 + T + window + D
    say(f"case window dtype={dtype} D={D} causal={causal} T={T} window={window} "
        f"globals={len(glob)} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    scale = default_scale(D)
    o, lse = run_window(x, causal, scale, window, glob)
    check(x, dtype, causal, scale, window, glob, o, lse, "small")


def test_window_token_list_forms():
    """Tokens as an int32 device tensor, with duplicates and positions outside
    [0, T) (ignored), give the same result as the clean list."""
    x = generate(1, 2, 1, 400, 64, "bf16", 9900)
    clean = (0, 17, 399)
    o1, l1 = run_window(x, True, 0.125, 40, clean)
    messy = torch.tensor([399, 17, 0, 17, -5, 400, 4000], dtype=torch.int32, device="cuda")
    o2, l2 = run_window(x, True, 0.125, 40, messy)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    check(x, "bf16", True, 0.125, 40, clean, o1, l1, "token forms")


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_everything_is_fwd_bitwise(causal):
    """window >= T - 1 without global tokens visits every tile with the same
    arithmetic as fa_fwd: bitwise the same output."""
    from exact_attention_91_amd import fa
    x = generate(2, 4, 2, 500, 64, "bf16", 9901)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    o1, l1 = fa.fwd(q, k, v, causal=causal, scale=0.125)
    o2, l2 = fa.fwd_window(q, k, v, 499, None, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_large_scores():
    x = generate(1, 4, 1, 700, 64, "bf16", 9902, qk_sigma=4.0)
    for causal in (False, True):
        o, lse = run_window(x, causal, 0.125, 50, (0, 350))
        check(x, "bf16", causal, 0.125, 50, (0, 350), o, lse, f"sigma4 causal={causal}")


def test_window_binding_errors():
    from exact_attention_91_amd import fa
    x = generate(1, 2, 1, 64, 64, "bf16", 9903)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    with pytest.raises(RuntimeError):
        fa.fwd_window(q, k, v, -1)
    with pytest.raises(TypeError):
        fa.fwd_window(q.float(), k.float(), v.float(), 8)
    with pytest.raises(ValueError):
        fa.fwd_window(q, k, v, 8, torch.tensor([1, 2], dtype=torch.int64, device="cuda"))


def test_workload_window():
    """B=2 H=12 T=8192 D=64, window 256 and tokens 0..15 global, causal:
    compared in full."""
    w = WORKLOADS["window"]
    say(f"workload {w.name}")
    x = generate_workload(w)
    o, lse = run_window(x, True, w.scale, w.window, w.global_tokens)
    check(x, w.dtype, True, w.scale, w.window, w.global_tokens, o, lse, w.name)


@pytest.mark.parametrize("T,tokens", [(1, [0]), (64, [63, 0, 63]), (65, [64]),
                                      (1000, list(range(3, 1000, 7)) + [-1, 1000, 5000]),
                                      (300, [])])
def test_window_bitmap_bits(T, tokens):
    """Bit j % 64 of word j // 64 is set iff j is a listed position in [0, T)."""
    from exact_attention_91_amd import fa
    bits = fa.window_bitmap(tokens, T, torch.device("cuda"))
    torch.cuda.synchronize()
    words = bits.cpu().numpy().view(np.uint64)
    expect = np.zeros((T + 63) // 64, np.uint64)
    for j in tokens:
        if 0 <= j < T:
            expect[j // 64] |= np.uint64(1) << np.uint64(j % 64)
    assert np.array_equal(words[:len(expect)], expect)


def test_window_prebuilt_bitmap_reused():
    """One bitmap serves several calls (two head groups, both masks) with the
    same result as building it per call."""
    from exact_attention_91_amd import fa
    glob = (0, 1, 200, 511)
    bits = fa.window_bitmap(glob, 512, torch.device("cuda"))
    for seed, causal in ((9904, True), (9905, False)):
        x = generate(1, 4, 2, 512, 64, "bf16", seed)
        q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
        o1, l1 = fa.fwd_window(q, k, v, 33, global_bits=bits, causal=causal, scale=0.125)
        o2, l2 = fa.fwd_window(q, k, v, 33, glob, causal=causal, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        check(x, "bf16", causal, 0.125, 33, glob, o1.double().cpu().numpy(),
              l1.double().cpu().numpy(), f"prebuilt causal={causal}")


# ---------------------------------------------------------------- backward

BWD_RTOL = {"bf16": 2e-2, "f16": 3e-3}   # as the plain backward (tests/test_gpu_bwd.py)


def run_bwd_window(x, do, causal, scale, window, glob, head_split=0):
    from exact_attention_91_amd import fa
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    bits = fa.window_bitmap(glob, q.shape[1], q.device)
    o, lse = fa.fwd_window(q, k, v, window, causal=causal, scale=scale, global_bits=bits)
    g = fa.bwd_window(q, k, v, o, lse, do.cuda(), window, causal=causal, scale=scale,
                      global_bits=bits, head_split=head_split)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in g)


def check_bwd(x, do64, dtype, causal, scale, window, glob, got, label=""):
    from oracle import oracle as orc
    valid = [int(g) for g in glob if 0 <= int(g) < x.q64.shape[1]]
    ref = orc.attention_bwd_masked(x.q64, x.k64, x.v64, do64, causal, scale, window, valid)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), name
        err = float(np.max(np.abs(g - r)))
        tol = BWD_RTOL[dtype] * max(1.0, float(np.max(np.abs(r))))
        say(f"  {label} {name}: max|err|={err:.3e} (tol {tol:.3e})")
        assert err <= tol, (name, err, tol)


BWD_CASES = [(65, 0, ()), (300, 63, (0, 64, 299)), (300, 1, ()), (1000, 100, (0, 1, 2, 3)),
             (777, 31, tuple(range(0, 777, 97))), (1000, 2000, ())]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,window,glob", BWD_CASES)
def test_bwd_window_small(dtype, D, causal, T, window, glob):
    from exact_attention_91_amd.inputs import generate_dout
    B, H, H_kv = (2, 3, 1) if T < 500 else (1, 2, 2)
    seed = 9950 + T + window + D
    say(f"case bwd window dtype={dtype} D={D} causal={causal} T={T} window={window} "
        f"globals={len(glob)} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    do, do64 = generate_dout(B, H, T, D, dtype, seed)
    scale = default_scale(D)
    got = run_bwd_window(x, do, causal, scale, window, glob)
    check_bwd(x, do64, dtype, causal, scale, window, glob, got, "small")


@pytest.mark.parametrize("head_split", [1, 4, 0])
def test_bwd_window_head_split(head_split):
    from exact_attention_91_amd.inputs import generate_dout
    x = generate(2, 8, 1, 500, 64, "bf16", 9990)
    do, do64 = generate_dout(2, 8, 500, 64, "bf16", 9990)
    for causal in (False, True):
        got = run_bwd_window(x, do, causal, 0.125, 70, (3, 250), head_split=head_split)
        check_bwd(x, do64, "bf16", causal, 0.125, 70, (3, 250), got, f"split={head_split}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_window_covering_everything_is_bwd_bitwise(causal):
    """A window covering every key without global tokens: the same tiles and
    arithmetic as fa_bwd, bitwise the same gradients."""
    from exact_attention_91_amd import fa
    from exact_attention_91_amd.inputs import generate_dout
    x = generate(2, 4, 2, 300, 64, "bf16", 9991)
    do = generate_dout(2, 4, 300, 64, "bf16", 9991)[0].cuda()
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.125)
    a = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=0.125, head_split=1)
    b = fa.bwd_window(q, k, v, o, lse, do, 299, causal=causal, scale=0.125, head_split=1)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_bwd_workload_window():
    """The window workload's backward (B=2 H=12 T=8192 D=64, window 256, tokens
    0..15 global, causal), compared in full."""
    from exact_attention_91_amd.inputs import generate_dout
    w = WORKLOADS["window"]
    say(f"workload bwd {w.name}")
    x = generate_workload(w)
    do, do64 = generate_dout(w.B, w.H, w.T, w.D, w.dtype, w.seed)
    got = run_bwd_window(x, do, True, w.scale, w.window, w.global_tokens)
    check_bwd(x, do64, w.dtype, True, w.scale, w.window, w.global_tokens, got, w.name)


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_window_scale_values(scale):
    """Negative scale (q's sign flipped in registers) and zero scale (uniform
    weights over each row's visible keys), forward and backward."""
    from exact_attention_91_amd.inputs import generate_dout
    x = generate(1, 4, 2, 300, 64, "bf16", 9995)
    do, do64 = generate_dout(1, 4, 300, 64, "bf16", 9995)
    for causal in (False, True):
        o, lse = run_window(x, causal, scale, 20, (0, 150))
        check(x, "bf16", causal, scale, 20, (0, 150), o, lse, f"scale={scale}")
        got = run_bwd_window(x, do, causal, scale, 20, (0, 150))
        check_bwd(x, do64, "bf16", causal, scale, 20, (0, 150), got, f"scale={scale}")
