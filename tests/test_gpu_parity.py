"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Small shapes are compared element by element and span several query/key tiles
with ragged tails; the full-size workloads run in the same launch
configuration the benchmark times and are compared in full where the oracle
finishes in seconds, else on seeded samples of rows.
"""
import numpy as np
import pytest
import torch

from exact_attention_91_amd.inputs import WORKLOADS, default_scale, generate, \
    generate_workload, sample_rows
from tests.gpu_util import TOL, check_full, check_rows, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL_T = [1, 7, 63, 64, 65, 127, 129, 300, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", SMALL_T)
def test_small_elementwise(dtype, D, causal, T):
    B, H, H_kv = (2, 3, 1) if T < 500 else (1, 2, 2)
    seed = 5000 + T * 10 + D
    say(f"case dtype={dtype} D={D} causal={causal} B={B} H={H} H_kv={H_kv} T={T} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    scale = default_scale(D)
    o, lse = run_gpu(x, causal, scale)
    check_full(x, dtype, causal, scale, o, lse, "small")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (6, 2), (8, 1)])
def test_kv_head_groups(dtype, H, H_kv):
    B, T, D = 2, 200, 64
    say(f"case groups dtype={dtype} H={H} H_kv={H_kv}")
    x = generate(B, H, H_kv, T, D, dtype, 77 + H * 10 + H_kv)
    for causal in (False, True):
        o, lse = run_gpu(x, causal, 0.125)
        check_full(x, dtype, causal, 0.125, o, lse, f"groups causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9, 1e-3])
def test_scale_values(dtype, scale):
    """Any finite scale: 0 gives uniform weights, negative flips the scores."""
    B, H, T, D = 1, 2, 150, 32
    say(f"case scale={scale} dtype={dtype}")
    x = generate(B, H, 1, T, D, dtype, 91)
    for causal in (False, True):
        o, lse = run_gpu(x, causal, scale)
        check_full(x, dtype, causal, scale, o, lse, f"scale={scale} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mag", [-1.0e9, 1.0e9])
@pytest.mark.parametrize("two_level", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 1)])
def test_scores_at_range_edge(dtype, mag, two_level, H, H_kv):
    """Scaled scores of magnitude up to 1e9, the edge of the documented range
    (|scale * q.k| < 1.4e9). At that size fp32 resolves scores only to ~64, so
    the inputs avoid near ties: key rows are one vector (every score of a row
    equal: uniform weights, O the (prefix) mean of V, L = s + ln n) or, with
    two_level, alternate between that vector and 1 + 2^-7 times it (scores
    differ by ~8e6: the larger level takes all the weight). The raw dot products
    are accumulated in fp32 (relative error up to D * 2^-24 = 3.8e-6 for
    D = 64) and L is stored in fp32, so L is judged against 1e-3 + 8e-6 |L|."""
    from exact_attention_91_amd.inputs import Inputs, _round
    B, T, D = 2, 300, 64
    say(f"case range edge dtype={dtype} mag={mag} two_level={two_level} H={H} H_kv={H_kv}")
    rng = np.random.default_rng(4243)
    kappa = 64.0
    a = rng.uniform(0.5, 1.0, size=(B, T, H, 1))
    # score = 0.125 * D * q * kappa * level  ->  q = mag * a / (0.125 * D * kappa)
    q = np.broadcast_to(a * mag / (0.125 * D * kappa), (B, T, H, D)).copy()
    k = np.full((B, T, H_kv, D), kappa)
    if two_level:
        k[:, 1::2] *= 1.0 + 2.0 ** -7
    v = rng.standard_normal((B, T, H_kv, D))
    qt, q64 = _round(q, dtype)
    kt, k64 = _round(k, dtype)
    vt, v64 = _round(v, dtype)
    scores = 0.125 * np.einsum("bthd,bshd->bhts", q64[:, :, :1], k64[:, :, :1])
    assert np.max(np.abs(scores)) < 1.4e9
    x = Inputs(q64, k64, v64, qt, kt, vt)
    from oracle import oracle as orc
    for causal in (False, True):
        o, lse = run_gpu(x, causal, 0.125)
        o_ref, l_ref = orc.attention(x.q64, x.k64, x.v64, causal, 0.125)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        eo = float(np.max(np.abs(o - o_ref)))
        rel_l = float(np.max(np.abs(lse - l_ref) / (1e-3 + 8e-6 * np.abs(l_ref))))
        say(f"  causal={causal} max|dO|={eo:.3e} max|dL|/(1e-3+8e-6|L|)={rel_l:.3e} "
            f"L range [{l_ref.min():.3e}, {l_ref.max():.3e}]")
        assert eo <= TOL[dtype][0]
        assert rel_l <= 1.0


@pytest.mark.parametrize("causal", [False, True])
def test_large_scores_rescaling(causal):
    """q, k ~ N(0, 4^2): scores of magnitude ~100 force many rescales."""
    B, H, T, D = 2, 4, 700, 64
    x = generate(B, H, 1, T, D, "bf16", 92, qk_sigma=4.0)
    o, lse = run_gpu(x, causal, 0.125)
    check_full(x, "bf16", causal, 0.125, o, lse, "sigma4")


# ---------------------------------------------------------------- full size

def test_workload_single_head_fp32():
    w = WORKLOADS["single_head_fp32"]
    x = generate_workload(w)
    for causal in w.causal:
        say(f"workload {w.name} causal={causal}")
        o, lse = run_gpu(x, causal, w.scale)
        check_full(x, w.dtype, causal, w.scale, o, lse, w.name)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_workload_batched(D):
    w = WORKLOADS[f"batched_d{D}"]
    say(f"workload {w.name}")
    x = generate_workload(w)
    o, lse = run_gpu(x, True, w.scale)
    check_full(x, w.dtype, True, w.scale, o, lse, w.name)


@pytest.mark.parametrize("name", ["gpt2", "gpt2_f16"])
def test_workload_gpt2(name):
    w = WORKLOADS[name]
    say(f"workload {w.name}")
    x = generate_workload(w)
    o, lse = run_gpu(x, True, w.scale)
    check_full(x, w.dtype, True, w.scale, o, lse, w.name)


def test_workload_long_sampled_rows():
    """256 seeded query rows per batch (edge rows included), full-row oracle."""
    w = WORKLOADS["long"]
    say(f"workload {w.name}")
    x = generate_workload(w)
    o, lse = run_gpu(x, True, w.scale)
    rows = sample_rows(w.B, w.H, w.T, 256, seed=w.seed + 7,
                       fixed=(0, 1, 63, 64, 127, 128, 4095, 4096, 8190, 8191))
    assert len(rows) == 256 * w.B
    check_rows(x, w.dtype, True, w.scale, o, lse, rows, w.name)
    # properties that hold at any size, checked on every row
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o)) <= np.max(np.abs(x.v64)) + TOL["bf16"][0]


def test_workload_mqa_full():
    """MQA (q, k ~ N(0, 4^2): near one-hot rows, frequent rescales), compared
    with the oracle on every one of its 393,216 rows."""
    w = WORKLOADS["mqa"]
    say(f"workload {w.name}")
    x = generate_workload(w)
    o, lse = run_gpu(x, True, w.scale)
    check_full(x, w.dtype, True, w.scale, o, lse, w.name)
    # O is a convex combination of V rows
    assert np.max(np.abs(o)) <= np.max(np.abs(x.v64)) + TOL["bf16"][0]


@pytest.mark.parametrize("B,T,D", [(5, 8000, 128), (4, 8192, 128), (16, 4200, 64)])
def test_two_group_long_rows(B, T, D):
    """Long causal rows with every work-group resident at once: each query
    tile's keys are split between two wave groups and merged in LDS. Odd
    key-tile counts (T = 8000 and 4200 end mid-tile) give group 1 one step
    less. Compared in full."""
    from exact_attention_91_amd import fa
    assert fa.key_groups(B, 1, T, D, torch.bfloat16) == 2
    say(f"case two groups B={B} T={T} D={D}")
    x = generate(B, 1, 1, T, D, "bf16", 9700 + T + D)
    scale = default_scale(D)
    o, lse = run_gpu(x, True, scale)
    check_full(x, "bf16", True, scale, o, lse, "two groups")


# Sizes with more query tiles than a quarter of the resident work-groups and
# short rows: the one-group kernel at D = 64 and 128, on ragged and tiny T.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 63, 65, 129, 300])
def test_one_group_ragged(dtype, D, causal, T):
    from exact_attention_91_amd import fa
    B, H = 16, 17
    assert fa.key_groups(B, H, T, D, torch.bfloat16) == 1
    seed = 9600 + T * 10 + D
    say(f"case one group dtype={dtype} D={D} causal={causal} B={B} H={H} T={T} seed={seed}")
    x = generate(B, H, 1, T, D, dtype, seed)
    scale = default_scale(D)
    o, lse = run_gpu(x, causal, scale)
    check_full(x, dtype, causal, scale, o, lse, "one group")


def _fwd_into_nan(q, k, v, causal, scale):
    """fa_fwd through the C ABI into outputs filled with NaN first, so a query
    tile that no work-group visits shows up in the comparison."""
    from exact_attention_91_amd import fa
    B, T, H, D = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device=q.device)
    rc = fa._lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr(), B, H, k.shape[2], T, D, int(causal), float(scale),
                          fa._dtype_code(q), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fa.status_str(rc)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


# Causal grids that are resident on the chip all at once, where the work-group
# order alternates direction per round of 256 (one work-group per CU per
# round): 550 one-group work-groups at D = 64, 512 head-pair work-groups
# (8 query heads per 2 kv heads), 512 one-group work-groups at D = 128 (fp16)
# and 512 fp32 work-groups. Outputs start as NaN, so a unit the permuted order
# skipped or visited twice in place of another fails.
@pytest.mark.parametrize("dtype,B,H,H_kv,T,D", [("bf16", 11, 5, 5, 1200, 64),
                                                ("bf16", 16, 8, 2, 1024, 64),
                                                ("f16", 64, 1, 1, 1024, 128),
                                                ("f32", 8, 8, 8, 1000, 32)])
def test_resident_grid_order(dtype, B, H, H_kv, T, D):
    seed = 9900 + B + H + T + D
    say(f"case resident order dtype={dtype} B={B} H={H} H_kv={H_kv} T={T} D={D} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    scale = default_scale(D)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    o, lse = _fwd_into_nan(q, k, v, True, scale)
    check_full(x, dtype, True, scale, o, lse, "resident order")
