"""Stream and graph behaviour of the C ABI (needs a GPU).

Every entry point enqueues on the stream it is given and allocates nothing,
so (a) work on a side stream is ordered by that stream and gives the same
bits as on the default stream, and (b) forward and backward can be captured
into a HIP graph and replayed. Each replay is checked against the eager
result, with eager work and synchronisations between replays.
"""

import pytest
import torch

from exact_io_aware_54_amd import inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)


def test_side_stream_matches_default(gpu_lib):
    B, H, N, d = 2, 4, 700, 128
    note(f"side stream bf16 B{B} H{H} N{N} d{d}")
    q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, 9101, torch.bfloat16,
                                                        with_do=True))
    o0, l0 = gpu_lib.forward(q, k, v, causal=True)
    g0 = gpu_lib.backward(q, k, v, o0, l0, do, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1 = torch.empty_like(q)
        l1 = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
        gpu_lib.fa_fwd(q, k, v, o1, l1, d ** -0.5, True, stream=side)
        dq1, dk1, dv1 = (torch.empty_like(q) for _ in range(3))
        ws = gpu_lib.workspace_for(q)
        gpu_lib.fa_bwd(q, k, v, o1, l1, do, dq1, dk1, dv1, ws, d ** -0.5, True, stream=side)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, (dq1, dk1, dv1)):
        assert torch.equal(a, b)


def test_graph_capture_and_replay(gpu_lib):
    B, H, N, d = 2, 4, 1000, 128
    note(f"graph capture fwd+bwd bf16 B{B} H{H} N{N} d{d}")
    q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, 9102, torch.bfloat16,
                                                        with_do=True))
    scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = gpu_lib.workspace_for(q)

    def step():
        gpu_lib.fa_fwd(q, k, v, o, lse, scale, True)
        gpu_lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, True)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((o, lse, dq, dk, dv), ref):
            assert torch.equal(got, exp), rep
