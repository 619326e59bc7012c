"""GPU parity on randomly drawn shapes: forward and backward against the
float64 oracle through the C ABI.

The parametrised tests elsewhere use hand-picked sequence lengths. Here a
fixed-seed generator draws the cases instead (N from 1 to 700, so ragged
tails at arbitrary offsets inside a 64-row tile; B*H from 1 to 6; every head
dim, dtype and mask; the softmax scale between 0.5 and 1.5 times 1/sqrt(d)),
so the case list is the same on every run and a failure names its case.
Tolerances are the suite's own (see test_parity_gpu):
  16-bit forward   O max-abs <= 2e-2 and relative Frobenius <= 1e-2,
                   LSE max-abs <= 1e-3
  16-bit backward  dQ, dK, dV max-abs <= 5e-2 and relative Frobenius <= 1e-2
  fp32 forward     O and LSE max-abs <= 1e-5
  fp8 forward      O relative Frobenius <= 5e-2 against the oracle on the
                   dequantised codes, LSE |error| <= 1e-3 * max(1, |LSE|)
                   (d = 128, the fp8 path's head dim; scale 1/sqrt(d))
The eight-wave forward, which fa_fwd picks only once a launch has a
workgroup per CU, is forced through fa_fwd_waves on the 16-bit cases it
supports (d <= 128) so that its ragged and causal edges are reached at these
small sizes too.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_54_amd import inputs
from tests.util import max_abs, rel_frob, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _draw_cases(n, seed, dtypes, dims):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(
            dtype=dtypes[int(rng.integers(len(dtypes)))],
            d=dims[int(rng.integers(len(dims)))],
            causal=bool(rng.integers(2)),
            B=int(rng.integers(1, 3)),
            H=int(rng.integers(1, 4)),
            N=int(rng.integers(1, 701)),
            scale_mul=float(rng.uniform(0.5, 1.5)),
            seed=20000 + i))
    return cases


CASES_16 = _draw_cases(28, 20261203, ["bf16", "f16"], [64, 128, 256])
CASES_32 = _draw_cases(8, 20261204, ["f32"], [64, 128])
CASES_8 = _draw_cases(8, 20261205, ["e4m3"], [128])


def _cid(c):
    return (f"{c['dtype']}-d{c['d']}-{'causal' if c['causal'] else 'full'}-"
            f"B{c['B']}H{c['H']}N{c['N']}")


def note(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(c):
    q, k, v, do = inputs.draw_qkv(c["B"], c["H"], c["N"], c["d"], c["seed"], DT[c["dtype"]],
                                  with_do=True)
    return q, k, v, do, c["scale_mul"] * c["d"] ** -0.5


@pytest.mark.parametrize("c", CASES_16, ids=_cid)
def test_random_shape_fwd_bwd(gpu_lib, c):
    note(f"random {_cid(c)} scale x{c['scale_mul']:.3f} seed={c['seed']}")
    q, k, v, do, scale = _inputs(c)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, lse = gpu_lib.forward(qg, kg, vg, scale=scale, causal=c["causal"])
    dq, dk, dv = gpu_lib.backward(qg, kg, vg, o, lse, dog, scale=scale, causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(to64(q), to64(k), to64(v), scale, c["causal"])
    assert max_abs(to64(o), o_ref) <= 2e-2
    assert rel_frob(to64(o), o_ref) <= 1e-2
    assert max_abs(to64(lse), l_ref) <= 1e-3
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), scale, c["causal"])
    for name, got, exp in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert max_abs(to64(got), exp) <= 5e-2, name
        assert rel_frob(to64(got), exp) <= 1e-2, name


@pytest.mark.parametrize("c", [c for c in CASES_16 if c["d"] <= 128][:6], ids=_cid)
def test_random_shape_fwd_eight_waves(gpu_lib, c):
    note(f"random eight-wave forward {_cid(c)} seed={c['seed']}")
    q, k, v, _, scale = _inputs(c)
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qg)
    lse = torch.empty((c["B"], c["H"], c["N"]), device="cuda", dtype=torch.float32)
    gpu_lib.fa_fwd_waves(qg, kg, vg, o, lse, scale, c["causal"], 8)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(to64(q), to64(k), to64(v), scale, c["causal"])
    assert max_abs(to64(o), o_ref) <= 2e-2
    assert rel_frob(to64(o), o_ref) <= 1e-2
    assert max_abs(to64(lse), l_ref) <= 1e-3


@pytest.mark.parametrize("c", CASES_32, ids=_cid)
def test_random_shape_fwd_f32(gpu_lib, c):
    note(f"random {_cid(c)} scale x{c['scale_mul']:.3f} seed={c['seed']}")
    q, k, v, _, scale = _inputs(c)
    o, lse = gpu_lib.forward(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(to64(q), to64(k), to64(v), scale, c["causal"])
    assert max_abs(to64(o), o_ref) <= 1e-5
    assert max_abs(to64(lse), l_ref) <= 1e-5


@pytest.mark.parametrize("c", CASES_8, ids=_cid)
def test_random_shape_fwd_fp8(gpu_lib, c):
    note(f"random {_cid(c)} seed={c['seed']}")
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    (q8, k8, v8), scales = inputs.draw_fp8(B, H, N, d, c["seed"])
    o, lse = gpu_lib.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), scales, scale=d ** -0.5,
                                 causal=c["causal"])
    torch.cuda.synchronize()
    q, k, v = [oracle.e4m3_decode(t.numpy()) * s for t, s in zip((q8, k8, v8), scales)]
    o_ref, l_ref = oracle.attention_forward(q, k, v, d ** -0.5, c["causal"])
    assert rel_frob(to64(o), o_ref) <= 5e-2
    err = np.max(np.abs(to64(lse) - l_ref) / np.maximum(1.0, np.abs(l_ref)))
    assert err <= 1e-3
