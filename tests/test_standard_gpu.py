"""GPU parity of the standard (materialising) attention baseline, fa_std_fwd.

The baseline writes S and P to memory (its own three kernels) and must give
the same O as the definition: it is checked against the float64 oracle with
the forward's tolerances (O max-abs <= 2e-2 and relative Frobenius <= 1e-2),
and against the fused forward on the same inputs. Its extra roundings (S and
P stored in the input type) stay inside those bounds: a score of magnitude
|S| rounded to bf16 moves P by about |S| * 2^-9 relatively.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_54_amd import inputs
from tests.util import max_abs, rel_frob, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def note(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 130, 300])
def test_std_small(gpu_lib, dtype, d, causal, N):
    note(f"std {dtype} B1 H3 N{N} d{d} causal={causal}")
    q, k, v = inputs.draw_qkv(1, 3, N, d, 5000 + N, DT[dtype])
    o = gpu_lib.forward_standard(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention_forward(to64(q), to64(k), to64(v), 1.0 / math.sqrt(d), causal)
    assert max_abs(to64(o), o_ref) <= 2e-2
    assert rel_frob(to64(o), o_ref) <= 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_std_matches_fused(gpu_lib, causal):
    B, H, N, d = 1, 4, 2048, 128
    note(f"std vs fused bf16 B{B} H{H} N{N} d{d} causal={causal}")
    q, k, v = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, 5101, torch.bfloat16))
    o_std = gpu_lib.forward_standard(q, k, v, causal=causal)
    o_fa, _ = gpu_lib.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    a, b = to64(o_std), to64(o_fa)
    assert np.all(np.isfinite(a))
    assert max_abs(a, b) <= 2e-2
    assert rel_frob(a, b) <= 1e-2


def test_std_exercise_shape(gpu_lib):
    """The pages' benchmark shape (B=1, H=32, d=128, fp16 random normals) at
    N = 8192, checked on sampled query rows of three heads."""
    B, H, N, d = 1, 32, 8192, 128
    note(f"std f16 B{B} H{H} N{N} d{d}")
    q, k, v = inputs.draw_qkv(B, H, N, d, 5102, torch.float16)
    o = gpu_lib.forward_standard(q.cuda(), k.cuda(), v.cuda(), causal=False)
    torch.cuda.synchronize()
    o64 = to64(o)
    assert np.all(np.isfinite(o64))
    rng = np.random.default_rng(5102)
    for h in (0, 17, 31):
        rows = np.unique(np.concatenate([[0, 1, N // 2, N - 1], rng.choice(N, 20, replace=False)]))
        o_ref, _ = oracle.attention_forward_rows(to64(q[0, h]), to64(k[0, h]), to64(v[0, h]),
                                                 rows, d ** -0.5, False)
        assert max_abs(o64[0, h, rows], o_ref) <= 2e-2, h
        assert rel_frob(o64[0, h, rows], o_ref) <= 1e-2, h
