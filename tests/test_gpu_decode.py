"""Decode-shaped forward (fa_fwd_decode) through the C ABI against the oracle's
decode attention: T_q query rows at the end of a T_k-long key/value cache
(query i sees keys j <= T_k - T_q + i when causal), compared element by
element. Cases cover one and several query rows, grouped and shared kv heads,
packed row tiles beyond one 128-row tile, ragged cache lengths, rows that see
no key (T_q > T_k), a single key, and key splits from 1 to 32 parts."""
import numpy as np
import pytest
import torch

from exact_attention_91_amd import fa
from exact_attention_91_amd.inputs import Inputs, _round
from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, H, H_kv, Tq, Tk, D, dtype, seed):
    rng = np.random.default_rng(seed)
    q, q64 = _round(rng.standard_normal((B, Tq, H, D)), dtype)
    k, k64 = _round(rng.standard_normal((B, Tk, H_kv, D)), dtype)
    v, v64 = _round(rng.standard_normal((B, Tk, H_kv, D)), dtype)
    return q, k, v, q64, k64, v64


def _check(B, H, H_kv, Tq, Tk, D, causal, nsplit, dtype, seed=0):
    from oracle import oracle as orc
    q, k, v, q64, k64, v64 = _inputs(B, H, H_kv, Tq, Tk, D, dtype, seed + Tq * 7 + Tk)
    scale = D ** -0.5
    o, lse = fa.fwd_decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale,
                           nsplit=nsplit)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    o_ref, l_ref = orc.attention_decode(q64, k64, v64, causal, scale)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin), "rows with no visible key differ"
    assert np.all(np.isfinite(o))
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[fin] - l_ref[fin]))) if fin.any() else 0.0
    say(f"  decode {dtype} B={B} H={H} H_kv={H_kv} Tq={Tq} Tk={Tk} D={D} causal={causal} "
        f"nsplit={nsplit}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL[dtype][0], f"O error {eo}"
    assert el <= TOL[dtype][1], f"L error {el}"
    return o, lse


CASES = [
    # B, H, H_kv, Tq, Tk, D, causal, nsplit
    (2, 8, 2, 1, 1000, 64, True, 4),
    (2, 8, 2, 1, 1000, 64, True, 1),
    (1, 12, 1, 1, 4096, 64, True, 16),     # shared kv head, one token
    (3, 4, 4, 7, 333, 128, True, 3),
    (2, 6, 3, 16, 65, 64, False, 2),
    (1, 32, 8, 5, 2000, 128, True, 8),
    (2, 4, 1, 130, 300, 64, True, 2),      # 520 packed rows: five row tiles
    (1, 2, 2, 10, 4, 64, True, 1),         # T_q > T_k: the first rows see no key
    (1, 2, 1, 3, 1, 16, True, 1),          # a single key
    (2, 8, 8, 64, 64, 32, True, 2),        # T_q = T_k: plain causal attention
    (1, 4, 2, 2, 700, 16, False, 32),      # more parts than some ranges can fill
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_matches_oracle(dtype, case):
    _check(*case, dtype)


def test_decode_long_cache_grouped_heads():
    """A grouped-head decode step against a 32768-token cache (8 query heads per
    kv head), the library's own split choice; compared in full."""
    B, H, H_kv, Tq, Tk, D = 2, 32, 4, 1, 32768, 128
    nsplit = fa.decode_splits(B, H_kv, H, Tq, Tk)
    assert nsplit > 1
    _check(B, H, H_kv, Tq, Tk, D, True, nsplit, "bf16", seed=5)


def test_decode_split_count_changes_only_rounding():
    """Results for 1 and 8 key parts agree within the bf16 tolerance (the
    partials are merged exactly up to fp32 rounding)."""
    o1, l1 = _check(2, 8, 2, 4, 3000, 64, True, 1, "bf16", seed=9)
    o8, l8 = _check(2, 8, 2, 4, 3000, 64, True, 8, "bf16", seed=9)
    assert np.max(np.abs(o1 - o8)) <= TOL["bf16"][0]
    assert np.max(np.abs(l1 - l8)) <= 1e-5


def test_decode_rows_equal_square_attention_rows():
    """With a cache whose earlier query rows are known, the decode rows equal
    the last T_q rows of fa_fwd on the full sequence, up to rounding."""
    B, H, H_kv, Tq, Tk, D = 2, 4, 2, 6, 200, 64
    rng = np.random.default_rng(31)
    qf, _ = _round(rng.standard_normal((B, Tk, H, D)), "bf16")
    k, _ = _round(rng.standard_normal((B, Tk, H_kv, D)), "bf16")
    v, _ = _round(rng.standard_normal((B, Tk, H_kv, D)), "bf16")
    of, lf = fa.fwd(qf.cuda(), k.cuda(), v.cuda(), causal=True, scale=0.125)
    od, ld = fa.fwd_decode(qf[:, Tk - Tq:].contiguous().cuda(), k.cuda(), v.cuda(), causal=True,
                           scale=0.125, nsplit=3)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(of[:, Tk - Tq:].float() - od.float())).item() <= 2 ** -7
    assert torch.max(torch.abs(lf[:, :, Tk - Tq:] - ld)).item() <= 1e-5
