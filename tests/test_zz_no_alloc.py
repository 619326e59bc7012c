"""GPU: fa_bwd_noalloc (the backward without a workspace argument, for callers
that cannot allocate) against fa_bwd through the C ABI.

Both run the same kernels on the same inputs, so their gradients must agree
bit for bit; the small case is also held to the oracle's bar (dQ, dK, dV
max-abs <= 5e-2 and relative Frobenius <= 1e-2). Two calls in a row, the
second on a smaller problem, then a third on new data, check that nothing of
an earlier call's scratch contents leaks into a later one; the last case fills
the scratch to its limit (B*H*N = 2^21 rows).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_54_amd import inputs
from tests.util import max_abs, rel_frob, to64

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)


def run_both(fa, B, H, N, d, causal, seed, dtype=torch.bfloat16, stream=None):
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, dtype, with_do=True))
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal)
    ref = fa.backward(q, k, v, o, lse, do, scale=scale, causal=causal)
    got = tuple(torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, o, lse, do, *got, scale, causal, stream=stream)
    torch.cuda.synchronize()
    return (q, k, v, do), ref, got


def test_noalloc_matches_fa_bwd_twice(gpu_lib):
    fa = gpu_lib
    note("noalloc: bf16 causal B2 H16 N2048 d128, then f16 B1 H3 N300 d64, then bf16 B1 H2 N129 d128")
    _, ref, got = run_both(fa, 2, 16, 2048, 128, True, 7101)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    (q, k, v, do), ref, got = run_both(fa, 1, 3, 300, 64, False, 7102, torch.float16)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    g_ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), 64 ** -0.5, False)
    for g, r in zip(got, g_ref):
        assert max_abs(to64(g), r) <= 5e-2
        assert rel_frob(to64(g), r) <= 1e-2
    _, ref, got = run_both(fa, 1, 2, 129, 128, True, 7103)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def test_noalloc_side_stream(gpu_lib):
    note("noalloc on a side stream: bf16 B1 H4 N1000 d64 causal")
    s = torch.cuda.Stream()
    _, ref, got = run_both(gpu_lib, 1, 4, 1000, 64, True, 7104, stream=s)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def test_noalloc_at_the_limit(gpu_lib):
    fa = gpu_lib
    B, H, N, d = 1, 64, 32768, 64
    assert B * H * N == fa.fa_bwd_noalloc_max_rows()
    note(f"noalloc at the scratch limit: bf16 causal B{B} H{H} N{N} d{d}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7105)
    q, k, v, do = (torch.randn((B, H, N, d), device="cuda", generator=gen).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.forward(q, k, v, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, causal=True)
    got = tuple(torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, o, lse, do, *got, d ** -0.5, True)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    with pytest.raises(fa.FAError) as exc:
        q2 = torch.empty((B, H, N + 1, d), device="cuda", dtype=torch.bfloat16)
        l2 = torch.empty((B, H, N + 1), device="cuda", dtype=torch.float32)
        fa.fa_bwd_noalloc(q2, q2, q2, q2, l2, q2, q2, q2, q2, d ** -0.5, True)
    assert exc.value.status == -8
    assert np.isfinite(to64(got[0][0, 0, :64])).all()


def test_noalloc_graph_capture(gpu_lib):
    """The callers it is for: forward + fa_bwd_noalloc captured into a HIP
    graph (through torch's capture) and replayed four times, with eager work
    between the replays that includes a different-size fa_bwd_noalloc call
    (which leaves its own contents in the shared scratch); every replay must
    give the eager result bit for bit."""
    fa = gpu_lib
    B, H, N, d = 2, 4, 1000, 128
    note(f"noalloc under graph capture: bf16 causal B{B} H{H} N{N} d{d}")
    q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, 7106, torch.bfloat16,
                                                        with_do=True))
    scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale, True)
        fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, True)

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
    # a different problem between replays, through the same scratch
    q2, k2, v2, do2 = (t.cuda() for t in inputs.draw_qkv(1, 3, 777, 64, 7107, torch.bfloat16,
                                                            with_do=True))
    o2, l2 = fa.forward(q2, k2, v2, causal=False)
    g2 = tuple(torch.empty_like(q2) for _ in range(3))
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        fa.fa_bwd_noalloc(q2, k2, v2, o2, l2, do2, *g2, 64 ** -0.5, False)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((o, lse, dq, dk, dv), ref):
            assert torch.equal(got, exp), rep
