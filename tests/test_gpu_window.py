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
    arithmetic as fa_fwd's one-group kernel: bitwise the same output (sizes
    for which fa_fwd picks that kernel)."""
    from exact_attention_91_amd import fa
    assert fa.key_groups(5, 16, 500, 64, torch.bfloat16) == 1
    x = generate(5, 16, 2, 500, 64, "bf16", 9901)
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
    arithmetic as fa_bwd, bitwise the same gradients. The sizes give fa_bwd's
    dQ kernel one wave group (240 query tiles of short rows at D = 64; on small
    grids it splits keys between two groups, which the window kernels do not)."""
    from exact_attention_91_amd import fa
    from exact_attention_91_amd.inputs import generate_dout
    x = generate(5, 16, 2, 300, 64, "bf16", 9991)
    do = generate_dout(5, 16, 300, 64, "bf16", 9991)[0].cuda()
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


# ------------------------------------- far queries of global key tiles split

def _bwd_pair(x, do, causal, scale, window, glob, head_split=0, n_global=None, n_split=None):
    """(split, unsplit) gradients: the split one with a workspace sized for
    n_global tokens (default: all of them), the unsplit one with fa_bwd's size.
    The split call leaves in the first header word past fa_bwd's workspace the
    number of global keys it served (n_split, default: all of them)."""
    from exact_attention_91_amd import fa
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    B, T, H, D = q.shape
    bits = fa.window_bitmap(glob, T, q.device)
    o, lse = fa.fwd_window(q, k, v, window, causal=causal, scale=scale, global_bits=bits)
    ng = len(set(glob)) if n_global is None else n_global
    ws = torch.empty((fa.bwd_window_workspace_bytes(B, H, k.shape[2], T, D, window, ng,
                                                     head_split),), dtype=torch.uint8,
                     device="cuda")
    ws0 = torch.empty((fa.bwd_workspace_bytes(B, H, k.shape[2], T, D, head_split),),
                      dtype=torch.uint8, device="cuda")
    a = fa.bwd_window(q, k, v, o, lse, do.cuda(), window, causal=causal, scale=scale,
                      global_bits=bits, head_split=head_split, workspace=ws)
    a2 = fa.bwd_window(q, k, v, o, lse, do.cuda(), window, causal=causal, scale=scale,
                       global_bits=bits, head_split=head_split, workspace=ws)
    u = fa.bwd_window(q, k, v, o, lse, do.cuda(), window, causal=causal, scale=scale,
                      global_bits=bits, head_split=head_split, workspace=ws0)
    torch.cuda.synchronize()
    for s, s2 in zip(a, a2):
        assert torch.equal(s, s2), "split backward not repeatable"
    base = fa.bwd_workspace_bytes(B, H, k.shape[2], T, D, head_split)
    served = int(ws[base:base + 4].cpu().view(torch.int32)[0])
    assert served == (len({g for g in glob if 0 <= g < T}) if n_split is None else n_split)
    return a, u


def _check_split(a, u, T, glob):
    """dQ and the rows of keys that are not global are bitwise those of the
    unsplit walk (the far queries add exact zeros there); the global keys'
    rows differ only in summation order."""
    assert torch.equal(a[0], u[0])
    gl = sorted({g for g in glob if 0 <= g < T})
    other = torch.ones(T, dtype=torch.bool)
    other[gl] = False
    for s, w in zip(a[1:], u[1:]):
        assert torch.equal(s[:, other.cuda()], w[:, other.cuda()])


SPLIT_CASES = [
    # T, window, globals, (B, H, H_kv), D
    (2000, 40, (0, 1, 7), (1, 2, 2), 64),
    (3000, 100, (5, 130, 131, 2999), (2, 2, 1), 64),
    (1500, 0, (700,), (1, 3, 3), 16),
    (1100, 64, (0, 500, 1099), (1, 4, 2), 128),
    (2600, 33, tuple(range(0, 2600, 301)), (1, 2, 1), 32),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,window,glob,heads,D", SPLIT_CASES)
def test_bwd_window_split(dtype, causal, T, window, glob, heads, D):
    from exact_attention_91_amd.inputs import generate_dout
    B, H, H_kv = heads
    seed = 12100 + T + D
    say(f"case bwd window split dtype={dtype} causal={causal} T={T} window={window} "
        f"globals={len(glob)} B={B} H={H} H_kv={H_kv} D={D} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    do, do64 = generate_dout(B, H, T, D, dtype, seed)
    scale = default_scale(D)
    a, u = _bwd_pair(x, do, causal, scale, window, glob)
    _check_split(a, u, T, glob)
    for g, label in ((a, "split"), (u, "unsplit")):
        got = tuple(t.double().cpu().numpy() for t in g)
        check_bwd(x, do64, dtype, causal, scale, window, glob, got, label)


@pytest.mark.parametrize("head_split", [1, 3, 0])
def test_bwd_window_split_with_head_split(head_split):
    """Grouped heads: the band part of each head part and the far chunks (all
    heads) add into the same global-key slots."""
    from exact_attention_91_amd.inputs import generate_dout
    B, H, H_kv, T, D = 2, 6, 1, 1800, 64
    glob = (0, 3, 900)
    x = generate(B, H, H_kv, T, D, "bf16", 12200 + head_split)
    do, do64 = generate_dout(B, H, T, D, "bf16", 12200 + head_split)
    for causal in (False, True):
        say(f"case bwd window split head_split={head_split} causal={causal}")
        a, u = _bwd_pair(x, do, causal, 0.125, 50, glob, head_split=head_split)
        _check_split(a, u, T, glob)
        got = tuple(t.double().cpu().numpy() for t in a)
        check_bwd(x, do64, "bf16", causal, 0.125, 50, glob, got, f"split hs={head_split}")


@pytest.mark.parametrize("n_global,n_split", [(1, 1), (2, 1), (3, 3), (4, 4), (5, 5)])
def test_bwd_window_split_too_few_slots(n_global, n_split):
    """A workspace with slots for fewer global keys than there are: the global
    tiles whose keys all have slots are split, the later ones keep the full
    walk; the result is the same either way."""
    from exact_attention_91_amd.inputs import generate_dout
    B, H, H_kv, T, D = 1, 2, 2, 2100, 64
    glob = (2, 300, 301, 1000, 2099)      # key tiles 0, 2, 2, 7, 16
    x = generate(B, H, H_kv, T, D, "bf16", 12300)
    do, do64 = generate_dout(B, H, T, D, "bf16", 12300)
    say(f"case bwd window split n_global={n_global}")
    a, u = _bwd_pair(x, do, True, 0.125, 30, glob, n_global=n_global, n_split=n_split)
    _check_split(a, u, T, glob)
    got = tuple(t.double().cpu().numpy() for t in a)
    check_bwd(x, do64, "bf16", True, 0.125, 30, glob, got, f"slots={n_global}")


def test_bwd_window_split_many_global_tiles():
    """More key tiles holding a global token than the split serves (64): the
    first 64 are split, the others keep the full walk."""
    from exact_attention_91_amd.inputs import generate_dout
    B, H, H_kv, T, D = 1, 1, 1, 128 * 70, 32
    glob = tuple(range(5, T, 128))       # one token in each of 70 key tiles
    x = generate(B, H, H_kv, T, D, "bf16", 12400)
    do, do64 = generate_dout(B, H, T, D, "bf16", 12400)
    say("case bwd window split 70 global tiles")
    a, u = _bwd_pair(x, do, True, default_scale(D), 16, glob, n_split=64)
    _check_split(a, u, T, glob)
    got = tuple(t.double().cpu().numpy() for t in a)
    check_bwd(x, do64, "bf16", True, default_scale(D), 16, glob, got, "70 tiles")
