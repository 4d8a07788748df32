"""Split-K forward and the logsumexp combine, through the C ABI, against the
float64 oracle.

fa_fwd_splitk must equal full attention (oracle.attention) to the same
tolerance as fa_fwd; the partials it leaves in the workspace must equal the
oracle's attention over each part's key range (oracle.attention_range); and
fa_lse_combine fed the oracle's own partials must reproduce full attention.
"""
import numpy as np
import pytest
import torch

from exact_attention_91_amd.inputs import WORKLOADS, default_scale, generate, \
    generate_workload, sample_rows
from tests.gpu_util import TOL, check_full, check_rows, max_err, say, to_gpu

pytestmark = pytest.mark.gpu

BQ, BK = 128, 64     # query rows per tile and keys per tile of the split kernel


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_splitk(x, causal, scale, nsplit, workspace=None):
    from exact_attention_91_amd import fa
    q, k, v = to_gpu(x)
    o, lse = fa.fwd_splitk(q, k, v, causal=causal, scale=scale, nsplit=nsplit,
                           workspace=workspace)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 65, 300, 1000])
@pytest.mark.parametrize("nsplit", [2, 7])
def test_splitk_elementwise(dtype, D, causal, T, nsplit):
    B, H, H_kv = (2, 3, 1) if T < 500 else (1, 2, 2)
    seed = 7000 + T * 10 + D + nsplit
    say(f"case splitk dtype={dtype} D={D} causal={causal} T={T} nsplit={nsplit} seed={seed}")
    x = generate(B, H, H_kv, T, D, dtype, seed)
    scale = default_scale(D)
    o, lse = run_splitk(x, causal, scale, nsplit)
    check_full(x, dtype, causal, scale, o, lse, "splitk")


@pytest.mark.parametrize("nsplit", [1, 3, 4, 16, 40])
def test_splitk_split_counts(nsplit):
    """1 (plain forward), counts that do not divide the key tiles, and counts
    above the number of key tiles (empty parts, -inf logsumexp)."""
    B, H, T, D = 1, 2, 777, 64
    x = generate(B, H, 1, T, D, "bf16", 7100 + nsplit)
    for causal in (False, True):
        say(f"case splitk nsplit={nsplit} causal={causal}")
        o, lse = run_splitk(x, causal, 0.125, nsplit)
        check_full(x, "bf16", causal, 0.125, o, lse, f"nsplit={nsplit} causal={causal}")


@pytest.mark.parametrize("H,H_kv", [(6, 2), (8, 1)])
def test_splitk_kv_groups(H, H_kv):
    x = generate(2, H, H_kv, 260, 64, "bf16", 7200 + H)
    for causal in (False, True):
        say(f"case splitk groups H={H} H_kv={H_kv} causal={causal}")
        o, lse = run_splitk(x, causal, 0.125, 3)
        check_full(x, "bf16", causal, 0.125, o, lse, "groups")


def test_splitk_large_scores():
    """Scores of magnitude ~100: each part has its own running max, so the
    combine must rescale parts whose logsumexps differ by hundreds."""
    x = generate(2, 2, 1, 700, 64, "bf16", 7300, qk_sigma=4.0)
    for causal in (False, True):
        o, lse = run_splitk(x, causal, 0.125, 4)
        check_full(x, "bf16", causal, 0.125, o, lse, f"sigma4 causal={causal}")


def _part_range(q0, T, causal, s, nsplit):
    kend = min(T, q0 + BQ) if causal else T
    n = (kend + BK - 1) // BK
    lo, hi = s * n // nsplit * BK, (s + 1) * n // nsplit * BK
    return lo, min(hi, kend)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nsplit", [3, 6])
def test_splitk_workspace_partials(causal, nsplit):
    """The workspace partials equal attention over each part's documented key
    range, normalised over that range (empty range: O_s = 0, L_s = -inf)."""
    from exact_attention_91_amd import fa
    from oracle import oracle as orc
    B, H, H_kv, T, D = 1, 2, 1, 400, 32
    x = generate(B, H, H_kv, T, D, "bf16", 7400 + nsplit)
    need = fa.splitk_workspace_bytes(B, H, T, D, nsplit)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    run_splitk(x, causal, 0.2, nsplit, workspace=ws)
    rows = B * H * T
    opart = ws[:rows * nsplit * D * 4].view(torch.float32).view(nsplit, B, H, T, D)
    lpart = ws[rows * nsplit * D * 4:].view(torch.float32).view(nsplit, B, H, T)
    opart = opart.double().cpu().numpy()
    lpart = lpart.double().cpu().numpy()
    for q0 in range(0, T, BQ):
        q1 = min(T, q0 + BQ)
        for s in range(nsplit):
            lo, hi = _part_range(q0, T, causal, s, nsplit)
            o_ref, l_ref = orc.attention_range(x.q64, x.k64, x.v64, causal, 0.2, lo, hi)
            o_ref, l_ref = o_ref[:, :, q0:q1], l_ref[:, :, q0:q1]
            og, lg = opart[s, :, :, q0:q1], lpart[s, :, :, q0:q1]
            empty = np.isneginf(l_ref)
            assert np.array_equal(np.isneginf(lg), empty), (q0, s)
            assert np.all(og[empty] == 0.0)
            eo = max_err(og[~empty], o_ref[~empty])
            el = max_err(lg[~empty], l_ref[~empty])
            say(f"  q0={q0} part={s} keys=[{lo},{hi}) dO={eo:.2e} dL={el:.2e}")
            assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1], (q0, s, eo, el)


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("nparts", [1, 2, 5])
def test_lse_combine_oracle_partials(out, nparts):
    """fa_lse_combine on the oracle's partials over a key partition (with an
    empty part when nparts = 5) reproduces full attention."""
    from exact_attention_91_amd import fa
    from oracle import oracle as orc
    B, H, T, D = 2, 3, 150, 64
    x = generate(B, H, H, T, D, "f32", 7500 + nparts)
    causal, scale = True, 0.125
    cuts = np.linspace(0, T, nparts + 1).round().astype(int)
    if nparts == 5:
        cuts = np.array([0, 40, 40, 90, 149, T])       # one empty part
    parts = [orc.attention_range(x.q64, x.k64, x.v64, causal, scale, int(a), int(b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    op = torch.tensor(np.stack([p[0] for p in parts]), dtype=torch.float32).cuda()
    lp = torch.tensor(np.stack([p[1] for p in parts]), dtype=torch.float32).cuda()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    o, lse = fa.lse_combine(op, lp, dtype=tdt)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    say(f"case combine out={out} nparts={nparts}")
    # the partials are rounded to fp32 before the merge, so fp32 output meets 1e-5
    tol = {"f32": (1e-5, 1e-5), "bf16": (TOL["bf16"][0], 1e-5), "f16": (TOL["f16"][0], 1e-5)}
    o_ref, l_ref = orc.attention(x.q64, x.k64, x.v64, causal, scale)
    eo, el = max_err(o, o_ref), max_err(lse, l_ref)
    say(f"  dO={eo:.2e} dL={el:.2e}")
    assert eo <= tol[out][0] and el <= tol[out][1]


def test_lse_combine_all_empty_rows():
    """Rows whose parts are all empty: O = 0, L = -inf; other rows unaffected."""
    from exact_attention_91_amd import fa
    n, B, H, T, D = 3, 1, 1, 4, 16
    g = torch.Generator().manual_seed(7600)
    op = torch.randn((n, B, H, T, D), generator=g)
    lp = torch.randn((n, B, H, T), generator=g)
    lp[:, 0, 0, 1] = -float("inf")
    op[:, 0, 0, 1] = 0.0
    lp[1, 0, 0, 2] = -float("inf")
    op[1, 0, 0, 2] = 0.0
    o, lse = fa.lse_combine(op.cuda(), lp.cuda(), dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.all(o[0, 1, 0] == 0.0) and np.isneginf(lse[0, 0, 1])
    from oracle import oracle as orc
    ro, rl = orc.lse_combine(op.double().numpy(), lp.double().numpy())
    for t in (0, 2, 3):
        assert max_err(o[0, t, 0], ro[0, 0, t]) <= 1e-5
        assert abs(lse[0, 0, t] - rl[0, 0, t]) <= 1e-5


def test_splitk_deterministic_and_workspace_reuse():
    """Two calls on one workspace (second one smaller) give bitwise the same
    result as calls on fresh workspaces."""
    from exact_attention_91_amd import fa
    xa = generate(2, 4, 2, 500, 64, "bf16", 7700)
    xb = generate(1, 2, 1, 130, 64, "bf16", 7701)
    ws = torch.empty((fa.splitk_workspace_bytes(2, 4, 500, 64, 5),), dtype=torch.uint8,
                     device="cuda")
    oa1, la1 = run_splitk(xa, True, 0.125, 5, workspace=ws)
    ob1, lb1 = run_splitk(xb, True, 0.125, 5, workspace=ws)
    oa2, la2 = run_splitk(xa, True, 0.125, 5)
    ob2, lb2 = run_splitk(xb, True, 0.125, 5)
    assert np.array_equal(oa1, oa2) and np.array_equal(la1, la2)
    assert np.array_equal(ob1, ob2) and np.array_equal(lb1, lb2)


def test_splitk_binding_errors():
    from exact_attention_91_amd import fa
    x = generate(1, 2, 1, 64, 64, "bf16", 7800)
    q, k, v = to_gpu(x)
    with pytest.raises(RuntimeError, match="workspace"):
        fa.fwd_splitk(q, k, v, nsplit=4,
                      workspace=torch.empty((64,), dtype=torch.uint8, device="cuda"))
    with pytest.raises(TypeError, match="bfloat16 or float16"):
        fa.fwd_splitk(q.float(), k.float(), v.float(), nsplit=2)
    with pytest.raises(RuntimeError):
        fa.fwd_splitk(q, k, v, nsplit=0)


# ---------------------------------------------------------------- full size

@pytest.mark.parametrize("nsplit", [2, 4])
def test_workload_long_splitk_sampled_rows(nsplit):
    w = WORKLOADS["long"]
    say(f"workload {w.name} splitk nsplit={nsplit}")
    x = generate_workload(w)
    o, lse = run_splitk(x, True, w.scale, nsplit)
    rows = sample_rows(w.B, w.H, w.T, 256, seed=w.seed + 9,
                       fixed=(0, 1, 63, 64, 127, 128, 4095, 4096, 8190, 8191))
    check_rows(x, w.dtype, True, w.scale, o, lse, rows, f"{w.name} nsplit={nsplit}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_workload_gpt2_splitk():
    w = WORKLOADS["gpt2"]
    say(f"workload {w.name} splitk nsplit=2")
    x = generate_workload(w)
    o, lse = run_splitk(x, True, w.scale, 2)
    check_full(x, w.dtype, True, w.scale, o, lse, f"{w.name} splitk")


@pytest.mark.parametrize("nsplit", [1, 4])
def test_workload_gpt2_b2(nsplit):
    """One GPU's share of gpt2 split by batch over 8 GPUs (192 work-groups)."""
    w = WORKLOADS["gpt2_b2"]
    say(f"workload {w.name} nsplit={nsplit}")
    x = generate_workload(w)
    o, lse = run_splitk(x, True, w.scale, nsplit)
    check_full(x, w.dtype, True, w.scale, o, lse, f"{w.name} nsplit={nsplit}")


@pytest.mark.parametrize("nsplit", [1, 8])
def test_workload_long_b1_sampled_rows(nsplit):
    """long at B=1 (64 work-groups unsplit), in the split the benchmark times."""
    w = WORKLOADS["long_b1"]
    say(f"workload {w.name} nsplit={nsplit}")
    x = generate_workload(w)
    o, lse = run_splitk(x, True, w.scale, nsplit)
    rows = sample_rows(w.B, w.H, w.T, 512, seed=w.seed + 7,
                       fixed=(0, 1, 63, 64, 127, 128, 1023, 1024, 4095, 4096, 8190, 8191))
    check_rows(x, w.dtype, True, w.scale, o, lse, rows, f"{w.name} nsplit={nsplit}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("B,H,T,D,nsplit", [(2, 4, 2000, 64, 4), (1, 1, 8192, 128, 8)])
def test_splitk_resident_grid_order(B, H, T, D, nsplit):
    """Key-split grids of 512 work-groups, all resident at once, whose order
    alternates direction per round of 256: with the workspace filled with NaN
    first, a (query tile, part) that no work-group visits would reach the
    output. Compared in full."""
    say(f"case splitk resident order B={B} H={H} T={T} D={D} nsplit={nsplit}")
    x = generate(B, H, H, T, D, "bf16", 7600 + T + D)
    from exact_attention_91_amd import fa
    need = fa.splitk_workspace_bytes(B, H, T, D, nsplit)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32,
                    device="cuda").view(torch.uint8)
    scale = default_scale(D)
    o, lse = run_splitk(x, True, scale, nsplit, workspace=ws)
    check_full(x, "bf16", True, scale, o, lse, f"resident order nsplit={nsplit}")
