"""Graph capture: the forward and backward, captured once in a HIP graph through
torch.cuda.graph, replay to the same bits as eager calls on the same inputs.

The kernels are deterministic (no atomics), launch on the caller's stream, issue
no memset and allocate nothing, so a replay must equal an eager call exactly.
Every replay is checked, with the inputs rewritten in place by eager work and a
synchronisation between replays."""
import math

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from exact_tiled_attention_34_amd import fa2  # noqa: E402


@pytest.mark.parametrize("d,causal", [(64, True), (128, False), (80, True), (256, True)])
def test_graph_replays_match_eager(d, causal):
    B, H, N = 2, 3, 300
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1234 + d)

    def fresh():
        return [torch.randn((B, H, N, d), device=dev, generator=gen).to(torch.bfloat16) for _ in range(4)]

    q, k, v, do = fresh()

    def step():
        o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
        dq, dk, dv = fa2.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
        return o, lse, dq, dk, dv

    # warm up on a side stream (library attributes cached, allocator pools primed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t, src in zip((q, k, v, do), fresh()):   # eager work between replays
            t.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = step()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), outs, want):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"
