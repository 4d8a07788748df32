"""The entry points under HIP graph capture: the library allocates nothing,
sets no memory and never synchronises, so a captured call replays like the
eager one. Each graph is replayed several times with the inputs rewritten
eagerly between replays (and the program's own work and synchronisation in
between); every replay must equal an eager call on the same inputs bitwise."""
import pytest
import torch

from exact_attention_91_amd.inputs import generate, generate_dout

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fresh(q, k, v, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in (q, k, v):
        t.copy_(torch.randn(t.shape, device="cuda", generator=g).to(t.dtype))


def _capture(fn):
    """Capture fn() on a side stream (warmed up first); return (graph, outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                     # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    torch.cuda.synchronize()
    return graph, out


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_graph_replays(causal):
    from exact_attention_91_amd import fa
    x = generate(2, 4, 2, 300, 64, "bf16", 12001)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    graph, (o, lse) = _capture(lambda: fa.fwd(q, k, v, causal=causal, scale=0.125))
    for rep in range(4):
        _fresh(q, k, v, 500 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el = fa.fwd(q, k, v, causal=causal, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), f"replay {rep}"


def test_bwd_and_splitk_and_window_graph_replays():
    """Forward, backward, key split, window forward and the window backward
    with its far split, captured in one graph."""
    from exact_attention_91_amd import fa
    B, H, H_kv, T, D = 1, 8, 2, 400, 64
    x = generate(B, H, H_kv, T, D, "bf16", 12002)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    do = generate_dout(B, H, T, D, "bf16", 12002)[0].cuda()
    bits = fa.window_bitmap((0, 7, 399), T, q.device)
    ws_b = torch.empty((fa.bwd_workspace_bytes(B, H, H_kv, T, D, 0),), dtype=torch.uint8,
                       device="cuda")
    ws_s = torch.empty((fa.splitk_workspace_bytes(B, H, T, D, 3),), dtype=torch.uint8,
                       device="cuda")
    # room for the 3 global keys' partial sums: the window backward's far split
    ws_w = torch.empty((fa.bwd_window_workspace_bytes(B, H, H_kv, T, D, 33, 3, 0),),
                       dtype=torch.uint8, device="cuda")

    def step():
        o, lse = fa.fwd(q, k, v, causal=True, scale=0.125)
        g = fa.bwd(q, k, v, o, lse, do, causal=True, scale=0.125, workspace=ws_b)
        os_, ls_ = fa.fwd_splitk(q, k, v, causal=True, scale=0.125, nsplit=3, workspace=ws_s)
        ow, lw = fa.fwd_window(q, k, v, 33, causal=True, scale=0.125, global_bits=bits)
        gw = fa.bwd_window(q, k, v, ow, lw, do, 33, causal=True, scale=0.125, global_bits=bits,
                           workspace=ws_w)
        return (o, lse) + tuple(g) + (os_, ls_, ow, lw) + tuple(gw)

    graph, outs = _capture(step)
    for rep in range(3):
        _fresh(q, k, v, 600 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {rep} output {i}"


_FIRST_CALL_CAPTURED = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from exact_attention_91_amd import fa
from exact_attention_91_amd.inputs import generate
x = generate(4, 8, 8, 1024, 64, "bf16", 12077)
q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    o, lse = fa.fwd(q, k, v, causal=True, scale=0.125)   # the library's first call
torch.cuda.synchronize()
for rep in range(3):
    g.replay()
    torch.cuda.synchronize()
    eo, el = fa.fwd(q, k, v, causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, eo) and torch.equal(lse, el), rep
print("first call captured: ok", flush=True)
"""


def test_fwd_first_call_under_capture():
    """A process whose first library call is made under graph capture (a
    causal grid: the launch then also asks the runtime, once per kernel, how
    many of its work-groups a CU holds): the capture succeeds and its replays
    equal eager calls. Runs in a child process, so no earlier call has done
    that query already."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED, root], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "first call captured: ok" in r.stdout
