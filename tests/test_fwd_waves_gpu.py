"""GPU tests of fa_fwd_waves: the forward with a forced workgroup shape.

Every wave handles 32 queries with the same per-query arithmetic whatever
the workgroup size, so the shapes must agree bit for bit with each other and
with fa_fwd; one small case per head dim is also checked against the
float64 oracle with the forward's tolerances (O max-abs <= 2e-2, relative
Frobenius <= 1e-2, LSE max-abs <= 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_54_amd import inputs
from tests.util import max_abs, rel_frob, to64

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)


def run(fa, q, k, v, causal, waves):
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    fa.fa_fwd_waves(q, k, v, o, lse, d ** -0.5, causal, waves)
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 200, 1000, 4096])
def test_shapes_bitwise_equal(gpu_lib, d, causal, N):
    note(f"fwd waves 0/4/8 bf16 B1 H3 N{N} d{d} causal={causal}")
    q, k, v = (t.cuda() for t in inputs.draw_qkv(1, 3, N, d, 8000 + N + d, torch.bfloat16))
    outs = [run(gpu_lib, q, k, v, causal, w) for w in (0, 4, 8)]
    o_ref, l_ref = gpu_lib.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


@pytest.mark.parametrize("d,waves", [(64, 8), (128, 4), (128, 8), (256, 4)])
def test_forced_shape_vs_oracle(gpu_lib, d, waves):
    N = 333
    note(f"fwd waves={waves} f16 B1 H2 N{N} d{d} causal=True")
    q, k, v = inputs.draw_qkv(1, 2, N, d, 8100 + d, torch.float16)
    o, lse = run(gpu_lib, q.cuda(), k.cuda(), v.cuda(), True, waves)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(to64(q), to64(k), to64(v), d ** -0.5, True)
    assert max_abs(to64(o), o_ref) <= 2e-2
    assert rel_frob(to64(o), o_ref) <= 1e-2
    assert max_abs(to64(lse), l_ref) <= 1e-3


def test_bad_shape_rejected(gpu_lib):
    q = torch.zeros(1, 1, 64, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.FAError):
        run(gpu_lib, q, q, q, False, 8)
    with pytest.raises(gpu_lib.FAError):
        run(gpu_lib, q[..., :128].contiguous(), q[..., :128].contiguous(),
            q[..., :128].contiguous(), False, 6)
