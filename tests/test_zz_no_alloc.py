"""The allocation-free key-split forward (fa_fwd_splitk_noalloc, partials in
the library's fixed device scratch) against the workspace entry point
fa_fwd_splitk on the same inputs, through the C ABI: bitwise equal (same
kernels, same key ranges) and within the bf16 tolerance of the oracle, on two
calls in a row, the second smaller, so stale scratch from the first call
would show."""
import pytest
import torch

from exact_attention_91_amd import fa
from exact_attention_91_amd.inputs import default_scale, generate
from tests.gpu_util import check_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [  # (B, H, H_kv, T, D, causal, nsplit): the second call is smaller
    (2, 4, 2, 3000, 128, True, 4),
    (1, 3, 1, 700, 64, True, 3),
]


def test_noalloc_equals_workspace_entry_point():
    for B, H, H_kv, T, D, causal, nsplit in CASES:
        need = fa.splitk_workspace_bytes(B, H, T, D, nsplit)
        assert 0 < need <= fa.splitk_scratch_bytes()
        say(f"case noalloc B={B} H={H} H_kv={H_kv} T={T} D={D} causal={causal} "
            f"nsplit={nsplit} partials={need} bytes")
        x = generate(B, H, H_kv, T, D, "bf16", 8800 + T + D)
        q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
        scale = default_scale(D)
        o2, l2 = fa.fwd_splitk_noalloc(q, k, v, causal=causal, scale=scale, nsplit=nsplit)
        torch.cuda.synchronize()
        o1, l1 = fa.fwd_splitk(q, k, v, causal=causal, scale=scale, nsplit=nsplit)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        check_full(x, "bf16", causal, scale, o2.double().cpu().numpy(),
                   l2.double().cpu().numpy(), "noalloc")


def test_noalloc_rejects_partials_beyond_scratch():
    B, H, T, D, nsplit = 4, 8, 8192, 128, 8
    assert fa.splitk_workspace_bytes(B, H, T, D, nsplit) > fa.splitk_scratch_bytes()
    q = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="fixed scratch"):
        fa.fwd_splitk_noalloc(q, q, q, causal=True, nsplit=nsplit)
