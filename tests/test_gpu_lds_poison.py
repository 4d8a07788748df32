"""The LDS-poisoning debug build (libfa_poison.so, compiled with
FA_LDS_POISON): every staged LDS buffer of the forward and backward kernels
holds NaN between the barrier that ends its last reads and its refill, so a
read that races a refill, or one that the tile barriers do not cover, turns
into NaN instead of silently reading stale data.

Every kernel family runs once through the debug build and once through the
release build on the same inputs; the outputs must be finite and bitwise
equal (the debug build adds fills and barriers, no arithmetic), and the
debug outputs are also compared with the float64 oracle on a few cases."""
import os

import pytest
import torch

from exact_attention_91_amd import build, fa
from exact_attention_91_amd.inputs import default_scale, generate, generate_dout
from tests.gpu_util import check_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(build.POISON_LIB):
        pytest.fail(f"{build.POISON_LIB} is missing: build() compiles it")


def both(fn):
    """fn() under the release build, then under the debug build."""
    a = fn()
    torch.cuda.synchronize()
    with fa.using_library(build.POISON_LIB):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b, label):
    for i, (x, y) in enumerate(zip(a, b)):
        assert bool(torch.isfinite(y).all()), f"{label}: output {i} of the debug build not finite"
        assert torch.equal(x, y), f"{label}: output {i} differs from the release build"
    say(f"  {label}: bitwise equal, finite")


def inputs(B, H, H_kv, T, D, dtype, seed, sigma=1.0):
    x = generate(B, H, H_kv, T, D, dtype, seed, qk_sigma=sigma)
    return x, x.q.cuda(), x.k.cuda(), x.v.cuda()


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_one_group(D, causal):
    """The plain forward (q and O through LDS), ragged T."""
    x, q, k, v = inputs(2, 3, 3, 1000, D, "bf16", 11 + D)
    a, b = both(lambda: fa.fwd(q, k, v, causal=causal, scale=default_scale(D)))
    same(a, b, f"fwd D={D} causal={causal}")
    if D == 64:
        check_full(x, "bf16", causal, default_scale(D), b[0].double().cpu().numpy(),
                   b[1].double().cpu().numpy(), "poison build vs oracle")


def test_forward_fp32():
    x, q, k, v = inputs(1, 2, 2, 300, 64, "f32", 12)
    a, b = both(lambda: fa.fwd(q, k, v, causal=True, scale=0.125))
    same(a, b, "fwd fp32")
    check_full(x, "f32", True, 0.125, b[0].double().cpu().numpy(), b[1].double().cpu().numpy(),
               "poison build vs oracle")


def test_forward_two_key_groups():
    """Long rows with few query tiles: the two-group (8-wave) kernel."""
    B, H, T, D = 1, 2, 4096, 128
    assert fa.key_groups(B, H, T, D, torch.bfloat16) == 2
    x, q, k, v = inputs(B, H, H, T, D, "bf16", 13)
    a, b = both(lambda: fa.fwd(q, k, v, causal=True, scale=default_scale(D)))
    same(a, b, "fwd two key groups")


def test_forward_head_pairs():
    """Query heads sharing a kv head: the head-pair (8-wave) kernel."""
    x, q, k, v = inputs(2, 4, 1, 500, 64, "bf16", 14, sigma=4.0)
    a, b = both(lambda: fa.fwd(q, k, v, causal=True, scale=0.125))
    same(a, b, "fwd head pairs")


def test_forward_window_splitk_decode():
    x, q, k, v = inputs(2, 4, 2, 900, 64, "bf16", 15)
    a, b = both(lambda: fa.fwd_window(q, k, v, 100, (0, 450), causal=True, scale=0.125))
    same(a, b, "window")
    a, b = both(lambda: fa.fwd_splitk(q, k, v, causal=True, scale=0.125, nsplit=3))
    same(a, b, "split-K")
    qd = q[:, -5:].contiguous()
    a, b = both(lambda: fa.fwd_decode(qd, k, v, causal=True, scale=0.125, nsplit=4))
    same(a, b, "decode")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward(D, causal):
    x, q, k, v = inputs(2, 4, 2, 700, D, "bf16", 16 + D)
    do = generate_dout(2, 4, 700, D, "bf16", 17)[0].cuda()
    o, lse = fa.fwd(q, k, v, causal=causal, scale=default_scale(D))
    a, b = both(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, scale=default_scale(D)))
    same(a, b, f"bwd D={D} causal={causal}")


@pytest.mark.parametrize("B,H,T,variant", [
    (16, 1, 4096, "K rows in LDS, 8 waves (512 key tiles)"),
    (16, 9, 500, "V rows in LDS, 32-row tiles"),
    (1, 17, 4096, "K and V in registers, 64-row tiles"),
])
def test_backward_d128_variants(B, H, T, variant):
    """The three D = 128 dK/dV kernels (the small cases above take the 8-wave
    one with K rows in LDS): more than 512 key-tile work-groups pick V rows in
    LDS, or with rows of at least 4096 keys K and V in registers."""
    D = 128
    x, q, k, v = inputs(B, H, H, T, D, "bf16", 20 + H)
    do = generate_dout(B, H, T, D, "bf16", 21 + H)[0].cuda()
    o, lse = fa.fwd(q, k, v, causal=True, scale=default_scale(D))
    a, b = both(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=default_scale(D)))
    same(a, b, f"bwd D=128 {variant}")


def test_backward_head_split_and_window():
    x, q, k, v = inputs(1, 12, 1, 600, 64, "bf16", 18)
    do = generate_dout(1, 12, 600, 64, "bf16", 19)[0].cuda()
    o, lse = fa.fwd(q, k, v, causal=True, scale=0.125)
    a, b = both(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=0.125, head_split=3))
    same(a, b, "bwd head split")
    ow, lw = fa.fwd_window(q, k, v, 64, (0, 300), causal=True, scale=0.125)
    a, b = both(lambda: fa.bwd_window(q, k, v, ow, lw, do, 64, (0, 300), causal=True,
                                      scale=0.125))
    same(a, b, "bwd window")
