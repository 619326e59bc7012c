"""GPU parity: libfa's kernels against the float64 CPU oracle (needs a gfx950 GPU).

Every call goes through the C ABI (via the ctypes binding). Inputs come from
the seeded generators in exact_io_aware_54_amd.inputs; the oracle receives
float64 copies of exactly the values the GPU received (for fp8: the E4M3
codes dequantised by the oracle's own decoder).

Tolerances (absolute errors are max over elements, "rel" is the relative
Frobenius error ||gpu - oracle|| / ||oracle||):
  fp32 forward         O max-abs <= 1e-5, LSE max-abs <= 1e-5
  bf16 / fp16 forward  O max-abs <= 2e-2 and rel <= 1e-2
  bf16 / fp16 backward dQ, dK, dV max-abs <= 5e-2 and rel <= 1e-2
  fp8 forward          O rel <= 5e-2
  LSE of the 16-bit path: max-abs <= 1e-3. The scores are exact products of
  the rounded inputs accumulated in fp32 and the row sum uses the unrounded
  fp32 probabilities, so LSE carries only fp32-level error (~1e-5); 1e-3
  leaves room for exp2/log2 approximations at N = 16K.
  LSE of the fp8 path: |error| <= 1e-3 * max(1, |LSE|). With the x20 outliers
  the scores reach |S| ~ 150, and the fp8 MFMA's score error alone reaches
  6.8e-4 of |S| (test_fwd_fp8_score_error: one key per head, where LSE = S
  exactly), so the bound scales with the magnitude.
Full-size workloads compare every element of sampled heads, or sampled query
rows computed one by one by the oracle (each output row depends only on its
own query row); properties that hold at any size are checked on all heads.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_54_amd import inputs
from tests.util import max_abs, rel_frob, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def note(msg):
    print(f"\n[case] {msg}", flush=True)


def dev(*ts):
    return tuple(t.cuda() for t in ts)


def check_fwd_full(fa, dtype, B, H, N, d, causal, seed, scale=None):
    note(f"fwd {dtype} B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = inputs.draw_qkv(B, H, N, d, seed, DT[dtype])
    o, lse = fa.forward(*dev(q, k, v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(to64(q), to64(k), to64(v), scale, causal)
    return to64(o), to64(lse), o_ref, l_ref


# ------------------------------------------------------------------ fp32 path

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,N", [(64, 128), (128, 77), (64, 1), (128, 200), (64, 300), (128, 513)])
def test_fwd_f32(gpu_lib, d, N, causal):
    seed = inputs.SEEDS["tiny_f32"] if (d, N) == (64, 128) else 2000 + N
    o, lse, o_ref, l_ref = check_fwd_full(gpu_lib, "f32", 1, 2, N, d, causal, seed)
    assert max_abs(o, o_ref) <= 1e-5
    assert max_abs(lse, l_ref) <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_f32_long(gpu_lib, causal):
    """fp32 over 128 key tiles per head in the eight-wave shape (B*H*N/256 =
    256 workgroups): sampled rows of four heads against the float64 oracle
    at the fp32 bound."""
    B, H, N, d = 1, 16, 4096, 128
    seed = 2100 + int(causal)
    note(f"fwd f32 B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    q, k, v = inputs.draw_qkv(B, H, N, d, seed, torch.float32)
    o, lse = gpu_lib.forward(*dev(q, k, v), scale=d ** -0.5, causal=causal)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    rng = np.random.default_rng(seed)
    for h in (0, 5, 10, 15):
        rows = _sample_rows(N, rng)
        o_ref, l_ref = oracle.attention_forward_rows(to64(q[0, h]), to64(k[0, h]), to64(v[0, h]),
                                                     rows, d ** -0.5, causal)
        assert max_abs(o64[0, h, rows], o_ref) <= 1e-5, h
        assert max_abs(l64[0, h, rows], l_ref) <= 1e-5, h


# ------------------------------------------------- 16-bit forward, small shapes

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 129, 300])
def test_fwd_16bit_small(gpu_lib, dtype, d, causal, N):
    o, lse, o_ref, l_ref = check_fwd_full(gpu_lib, dtype, 1, 3, N, d, causal, 3000 + N)
    assert max_abs(o, o_ref) <= 2e-2
    assert rel_frob(o, o_ref) <= 1e-2
    assert max_abs(lse, l_ref) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 300])
def test_fwd_d256_small(gpu_lib, dtype, causal, N):
    o, lse, o_ref, l_ref = check_fwd_full(gpu_lib, dtype, 1, 3, N, 256, causal, 3500 + N)
    assert max_abs(o, o_ref) <= 2e-2
    assert rel_frob(o, o_ref) <= 1e-2
    assert max_abs(lse, l_ref) <= 1e-3


def test_fwd_d256_workload(gpu_lib):
    """Head dim 256 (the largest the pages' SDPA interface takes), causal, N = 4096."""
    B, H, N, d = 1, 16, 4096, 256
    note(f"fwd bf16 causal B{B} H{H} N{N} d{d}")
    q, k, v = inputs.draw_qkv(B, H, N, d, 3601, torch.bfloat16)
    o, lse = gpu_lib.forward(*dev(q, k, v), causal=True)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(l64))
    rng = np.random.default_rng(3601)
    for h in (0, 9, 15):
        rows = _sample_rows(N, rng)
        o_ref, l_ref = oracle.attention_forward_rows(to64(q[0, h]), to64(k[0, h]), to64(v[0, h]),
                                                     rows, d ** -0.5, True)
        assert max_abs(o64[0, h, rows], o_ref) <= 2e-2, h
        assert rel_frob(o64[0, h, rows], o_ref) <= 1e-2, h
        assert max_abs(l64[0, h, rows], l_ref) <= 1e-3, h


def test_fwd_scale_argument(gpu_lib):
    """A scale other than 1/sqrt(d) reaches the scores (sharp softmax)."""
    o, lse, o_ref, l_ref = check_fwd_full(gpu_lib, "bf16", 1, 2, 200, 64, True, 3999, scale=0.9)
    assert max_abs(o, o_ref) <= 2e-2 and rel_frob(o, o_ref) <= 1e-2
    assert max_abs(lse, l_ref) <= 1e-3


# --------------------------------------------- 16-bit forward, full workloads

def _convex_hull_ok(o, v):
    """Each O row is a convex combination of V rows: column-wise within V's range."""
    lo = v.min(axis=-2, keepdims=True)
    hi = v.max(axis=-2, keepdims=True)
    tol = 1e-2 * np.maximum(np.abs(lo), np.abs(hi)) + 1e-3
    return bool(np.all(o >= lo - tol) and np.all(o <= hi + tol))


@pytest.mark.parametrize("N,seed", [(2048, inputs.SEEDS["fwd_bf16"]),
                                    (2000, inputs.SEEDS["fwd_bf16_ragged"])])
def test_fwd_bf16_d64_workload(gpu_lib, N, seed):
    B, H, d = 4, 16, 64
    note(f"fwd bf16 B{B} H{H} N{N} d{d} non-causal seed={seed}")
    q, k, v = inputs.draw_qkv(B, H, N, d, seed, torch.bfloat16)
    o, lse = gpu_lib.forward(*dev(q, k, v), scale=d ** -0.5, causal=False)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(l64))
    assert _convex_hull_ok(o64, to64(v))
    for b, h in [(0, 0), (1, 7), (3, 15)]:
        o_ref, l_ref = oracle.attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                                d ** -0.5, False)
        assert max_abs(o64[b, h], o_ref) <= 2e-2, (b, h)
        assert rel_frob(o64[b, h], o_ref) <= 1e-2, (b, h)
        assert max_abs(l64[b, h], l_ref) <= 1e-3, (b, h)


def _sample_rows(n, rng, extra=24):
    fixed = [0, 1, 2, 63, 64, 127, 128, 129, n // 2 + 17, n - 129, n - 65, n - 2, n - 1]
    rnd = rng.choice(n, size=extra, replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rnd]), 0, n - 1))


@pytest.mark.parametrize("N,seed,dtype", [(8192, inputs.SEEDS["causal_8k"], "bf16"),
                                          (16384, inputs.SEEDS["causal_16k"], "bf16"),
                                          (8192, inputs.SEEDS["causal_8k"], "f16")])
def test_fwd_bf16_causal_long(gpu_lib, N, seed, dtype):
    B, H, d = 1, 32, 128
    note(f"fwd {dtype} causal B{B} H{H} N{N} d{d} seed={seed}")
    q, k, v = inputs.draw_qkv(B, H, N, d, seed, DT[dtype])
    o, lse = gpu_lib.forward(*dev(q, k, v), scale=d ** -0.5, causal=True)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(l64))
    rng = np.random.default_rng(seed)
    for h in (0, 13, 31):
        rows = _sample_rows(N, rng)
        o_ref, l_ref = oracle.attention_forward_rows(to64(q[0, h]), to64(k[0, h]), to64(v[0, h]),
                                                     rows, d ** -0.5, True)
        assert max_abs(o64[0, h, rows], o_ref) <= 2e-2, h
        assert rel_frob(o64[0, h, rows], o_ref) <= 1e-2, h
        assert max_abs(l64[0, h, rows], l_ref) <= 1e-3, h
    # causal row 0 attends to key 0 only: O_0 = V_0 exactly (P = 1 is exact)
    assert np.array_equal(o64[0, :, 0], to64(v[0, :, 0]))


# ------------------------------------------------------------------ backward

def check_bwd_full(fa, dtype, B, H, N, d, causal, seed):
    note(f"bwd {dtype} B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = inputs.draw_qkv(B, H, N, d, seed, DT[dtype], with_do=True)
    qd, kd, vd, dod = dev(q, k, v, do)
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), scale, causal)
    return (to64(dq), to64(dk), to64(dv)), ref


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 130, 300])
def test_bwd_16bit_small(gpu_lib, dtype, d, causal, N):
    got, ref = check_bwd_full(gpu_lib, dtype, 1, 2, N, d, causal, 4000 + N)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert max_abs(g, r) <= 5e-2, name
        assert rel_frob(g, r) <= 1e-2, name


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 130, 300])
def test_bwd_d256_small(gpu_lib, dtype, causal, N):
    d = 256
    (dq, dk, dv), ref = check_bwd_full(gpu_lib, dtype, 1, 2, N, d, causal, 8500 + N)
    for got, exp in zip((dq, dk, dv), ref):
        assert max_abs(got, exp) <= 5e-2
        assert rel_frob(got, exp) <= 1e-2


def test_bwd_d256_noncausal_ragged(gpu_lib):
    """Head dim 256 without the mask over many tiles with a ragged end (N = 1000:
    15 full 64-row tiles and one of 40): the dQ pass takes the two 32-key halves
    one after the other there, and every Q / dO load of the split dK / dV
    launches and the ragged K / V loads use 32-bit offsets from the head base."""
    B, H, N, d = 1, 4, 1000, 256
    note(f"bwd bf16 non-causal B{B} H{H} N{N} d{d}")
    (dq, dk, dv), ref = check_bwd_full(gpu_lib, "bf16", B, H, N, d, False, 8700)
    for got, exp in zip((dq, dk, dv), ref):
        assert max_abs(got, exp) <= 5e-2
        assert rel_frob(got, exp) <= 1e-2


def test_bwd_d256_workload(gpu_lib):
    """Head dim 256 backward at a training-like shape, every element of two heads."""
    B, H, N, d = 2, 8, 2048, 256
    note(f"bwd bf16 causal B{B} H{H} N{N} d{d}")
    q, k, v, do = inputs.draw_qkv(B, H, N, d, 8601, torch.bfloat16, with_do=True)
    qg, kg, vg, dog = dev(q, k, v, do)
    o, lse = gpu_lib.forward(qg, kg, vg, causal=True)
    dq, dk, dv = gpu_lib.backward(qg, kg, vg, o, lse, dog, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for b, h in ((0, 0), (1, 7)):
        ref = oracle.attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                        to64(do[b, h]), d ** -0.5, True)
        for got, exp in zip((dq, dk, dv), ref):
            assert max_abs(to64(got[b, h]), exp) <= 5e-2, (b, h)
            assert rel_frob(to64(got[b, h]), exp) <= 1e-2, (b, h)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_noncausal_wide_launch(gpu_lib, d):
    """Non-causal backward on a launch large enough (B*H*ceil(N/256) >= 256)
    that the dQ pass takes its eight-wave workgroup shape: every element of
    three whole heads against the oracle."""
    B, H, N = 4, 16, 2048
    assert B * H * ((N + 255) // 256) >= 256
    seed = 4700 + d
    note(f"bwd bf16 non-causal B{B} H{H} N{N} d{d} seed={seed}")
    q, k, v, do = inputs.draw_qkv(B, H, N, d, seed, torch.bfloat16, with_do=True)
    qg, kg, vg, dog = dev(q, k, v, do)
    o, lse = gpu_lib.forward(qg, kg, vg, causal=False)
    dq, dk, dv = gpu_lib.backward(qg, kg, vg, o, lse, dog, causal=False)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for b, h in ((0, 0), (2, 9), (3, 15)):
        ref = oracle.attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                        to64(do[b, h]), d ** -0.5, False)
        for name, got, exp in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert max_abs(to64(got[b, h]), exp) <= 5e-2, (name, b, h)
            assert rel_frob(to64(got[b, h]), exp) <= 1e-2, (name, b, h)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fwd_bwd_training_workload(gpu_lib, dtype):
    """B8 H16 N4096 d128 causal: the shape the benchmark times (bf16), and the
    same launch configuration with fp16 inputs."""
    B, H, N, d = 8, 16, 4096, 128
    seed = inputs.SEEDS["train_4k"]
    scale = d ** -0.5
    note(f"fwd+bwd {dtype} causal B{B} H{H} N{N} d{d} seed={seed}")
    q, k, v, do = inputs.draw_qkv(B, H, N, d, seed, DT[dtype], with_do=True)
    qd, kd, vd, dod = dev(q, k, v, do)
    o, lse = gpu_lib.forward(qd, kd, vd, scale=scale, causal=True)
    dq, dk, dv = gpu_lib.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=True)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    grads = [to64(t) for t in (dq, dk, dv)]
    for t in [o64, l64] + grads:
        assert np.all(np.isfinite(t))
    # invariants at full size, every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    dk_sum = grads[1].sum(axis=2)
    assert np.max(np.abs(dk_sum)) <= 0.05 * np.sqrt(N)
    dv_sum, do_sum = grads[2].sum(axis=2), to64(do).sum(axis=2)
    assert rel_frob(dv_sum, do_sum) <= 1e-2
    for b, h in [(0, 0), (7, 15)]:
        o_ref, l_ref = oracle.attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                                scale, True)
        assert max_abs(o64[b, h], o_ref) <= 2e-2 and rel_frob(o64[b, h], o_ref) <= 1e-2
        assert max_abs(l64[b, h], l_ref) <= 1e-3
        ref = oracle.attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                        to64(do[b, h]), scale, True)
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            assert max_abs(g[b, h], r) <= 5e-2, (name, b, h)
            assert rel_frob(g[b, h], r) <= 1e-2, (name, b, h)


def test_bwd_stages_equal_bwd(gpu_lib):
    B, H, N, d = 1, 2, 300, 128
    note("fa_bwd_stage 1,2,3 vs fa_bwd")
    q, k, v, do = dev(*inputs.draw_qkv(B, H, N, d, 4444, torch.bfloat16, with_do=True))
    o, lse = gpu_lib.forward(q, k, v, scale=d ** -0.5, causal=True)
    dq1, dk1, dv1 = gpu_lib.backward(q, k, v, o, lse, do, scale=d ** -0.5, causal=True)
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = gpu_lib.workspace_for(q)
    for stage in (1, 2, 3):
        gpu_lib.fa_bwd_stage(stage, q, k, v, o, lse, do, dq2, dk2, dv2, ws, d ** -0.5, True)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


def test_determinism(gpu_lib):
    B, H, N, d = 2, 4, 1000, 128
    note("determinism")
    q, k, v, do = dev(*inputs.draw_qkv(B, H, N, d, 5555, torch.bfloat16, with_do=True))
    o1, l1 = gpu_lib.forward(q, k, v, causal=True)
    o2, l2 = gpu_lib.forward(q, k, v, causal=True)
    dq1, dk1, dv1 = gpu_lib.backward(q, k, v, o1, l1, do, causal=True)
    dq2, dk2, dv2 = gpu_lib.backward(q, k, v, o1, l1, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


# ------------------------------------------------------------------ closed forms

def test_closed_forms_gpu(gpu_lib):
    note("closed forms")
    d = 128
    g = torch.Generator().manual_seed(77)
    # one key: O = V_0, LSE = scale q.k
    q, k, v = (torch.randn(1, 2, 1, d, generator=g).to(torch.bfloat16) for _ in range(3))
    o, lse = gpu_lib.forward(*dev(q, k, v), scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), v)
    want = 0.1 * (to64(q) * to64(k)).sum(-1)
    assert max_abs(to64(lse), want) <= 1e-4
    # constant V: every output row equals that row (up to rounding P to bf16)
    N = 777
    q, k = (torch.randn(1, 2, N, d, generator=g).to(torch.bfloat16) for _ in range(2))
    row = torch.randn(d, generator=g).to(torch.bfloat16)
    v = row.expand(1, 2, N, d).contiguous()
    for causal in (False, True):
        o, _ = gpu_lib.forward(*dev(q, k, v), causal=causal)
        torch.cuda.synchronize()
        assert max_abs(to64(o), to64(v)) <= 2e-2
    # Q = 0: uniform weights, LSE = ln N (non-causal) and ln(i + 1) (causal)
    z = torch.zeros(1, 1, N, d, dtype=torch.bfloat16)
    v = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    o, lse = gpu_lib.forward(*dev(z, k[:, :1].contiguous(), v), causal=True)
    torch.cuda.synchronize()
    assert max_abs(to64(lse)[0, 0], np.log(np.arange(1, N + 1))) <= 1e-4
    cm = np.cumsum(to64(v)[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert max_abs(to64(o)[0, 0], cm) <= 2e-2


# ------------------------------------------------------------------ fp8 forward

def lse_rel_err(got, ref):
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))


def fp8_case(fa, B, H, N, d, causal, seed):
    note(f"fwd fp8 B{B} H{H} N{N} d{d} causal={causal} seed={seed}")
    (q8, k8, v8), scales = inputs.draw_fp8(B, H, N, d, seed)
    o, lse = fa.forward_fp8(*dev(q8, k8, v8), scales, scale=d ** -0.5, causal=causal)
    torch.cuda.synchronize()
    deq = [oracle.e4m3_decode(t.numpy()) * s for t, s in zip((q8, k8, v8), scales)]
    return to64(o), to64(lse), deq


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 300])
def test_fwd_fp8_small(gpu_lib, N, causal):
    o, lse, (q, k, v) = fp8_case(gpu_lib, 1, 2, N, 128, causal, 6000 + N)
    o_ref, l_ref = oracle.attention_forward(q, k, v, 128 ** -0.5, causal)
    assert rel_frob(o, o_ref) <= 5e-2
    assert lse_rel_err(lse, l_ref) <= 1e-3


def test_fwd_fp8_score_error(gpu_lib):
    """Evidence for the fp8 LSE bound. With a single key per head (N = 1) the
    softmax is trivial: LSE = S = scale * s_q * s_k * sum_d q8 k8 exactly,
    computed here in float64 from the decoded codes, so the kernel's LSE
    error is the score error of the fp8 MFMA (plus float32 rounding of the
    scale product and of exp2/log2 at p = 1). 8192 heads with the fp8
    workload's recipe (1 % x20 outliers) give scores up to |S| ~ 150.
    Measured on MI355X: max |error| / max(1, |S|) = 6.8e-4 (0.022 at
    |S| = 153), median 1.4e-5 -- far above float32 accumulation of 128 exact
    products (~1e-6), so the fp8 MFMA's internal sums are coarser than fp32.
    The fp8 tests' LSE bound, 1e-3 * max(1, |LSE|), is that score error with
    ~1.5x headroom; this test holds it to the same bound."""
    B, H, N, d = 1, 8192, 1, 128
    note(f"fp8 score error, one key per head B{B} H{H} N{N} d{d}")
    (q8, k8, v8), sc = inputs.draw_fp8(B, H, N, d, 6300)
    o, lse = gpu_lib.forward_fp8(*dev(q8, k8, v8), sc, scale=d ** -0.5, causal=False)
    torch.cuda.synchronize()
    q = oracle.e4m3_decode(q8.numpy()) * sc[0]
    k = oracle.e4m3_decode(k8.numpy()) * sc[1]
    s_ref = (q * k).sum(-1)[..., 0] * d ** -0.5            # [B, H]: one score per head
    err = np.abs(to64(lse)[..., 0] - s_ref)
    rel = err / np.maximum(1.0, np.abs(s_ref))
    print(f"[fp8 score error] max |S| {np.abs(s_ref).max():.1f}, max abs err {err.max():.3e}, "
          f"max err / max(1,|S|) {rel.max():.3e}, median {np.median(rel):.3e}", flush=True)
    assert rel.max() <= 1e-3
    # O of a single key is that key's V row (P = 1 exactly)
    v = oracle.e4m3_decode(v8.numpy()) * sc[2]
    assert rel_frob(to64(o), v) <= 5e-3


def _to_e4m3(x):
    """Per-tensor amax / 448 scaling and a round-to-nearest-even E4M3 cast."""
    s = float(x.abs().max() / 448.0)
    return (x / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8), s


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [128 ** -0.5, 0.5])
def test_fwd_fp8_growing_scores(gpu_lib, causal, scale):
    """Key norms ramp up along the sequence, so a row's max keeps growing and
    the running reference max is refreshed many times (by large steps at
    scale 0.5); O and LSE must still match the oracle on the dequantised
    inputs."""
    B, H, N, d = 1, 2, 1500, 128
    note(f"fwd fp8 ramped keys B{B} H{H} N{N} d{d} scale={scale:.4f} causal={causal}")
    gen = torch.Generator().manual_seed(6200 + int(causal))
    q = torch.randn(B, H, N, d, generator=gen)
    k = torch.randn(B, H, N, d, generator=gen) * torch.linspace(0.05, 2.0, N).view(1, 1, N, 1)
    v = torch.randn(B, H, N, d, generator=gen)
    (q8, sq), (k8, sk), (v8, sv) = (_to_e4m3(t) for t in (q, k, v))
    o, lse = gpu_lib.forward_fp8(*dev(q8, k8, v8), (sq, sk, sv), scale=scale, causal=causal)
    torch.cuda.synchronize()
    deq = [oracle.e4m3_decode(t.numpy()) * s for t, s in zip((q8, k8, v8), (sq, sk, sv))]
    o_ref, l_ref = oracle.attention_forward(*deq, scale, causal)
    assert np.all(np.isfinite(to64(o)))
    assert rel_frob(to64(o), o_ref) <= 5e-2
    assert lse_rel_err(to64(lse), l_ref) <= 1e-3


def test_fwd_fp8_max_size(gpu_lib):
    """The fp8 forward at B*H*N*d just below 2^31 (the ABI's limit): K/V tile
    offsets and head bases cross 2^30 bytes. E4M3 inputs are quantised on the
    device from a seeded generator (per-tensor amax / 448, round to nearest
    even); a first, a middle and the last head are checked against the oracle
    on the decoded codes, all outputs for finiteness."""
    B, H, N, d = 511, 32, 1024, 128
    assert 2 ** 30 + 2 ** 29 < B * H * N * d < 2 ** 31
    note(f"max size fp8 B{B} H{H} N{N} d{d} non-causal")
    g = torch.Generator(device="cuda")
    g.manual_seed(9101)
    codes, scales = [], []
    for _ in range(3):
        x = torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32)
        s = float(x.abs().max() / 448.0)
        codes.append((x / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
        scales.append(s)
        del x
    o, lse = gpu_lib.forward_fp8(*codes, tuple(scales), scale=d ** -0.5, causal=False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    for b, h in ((0, 0), (B // 2, 17), (B - 1, H - 1)):
        deq = [oracle.e4m3_decode(c[b, h].cpu().numpy()) * sc for c, sc in zip(codes, scales)]
        o_ref, l_ref = oracle.attention_forward(*deq, d ** -0.5, False)
        assert rel_frob(to64(o[b, h]), o_ref) <= 5e-2, (b, h)
        assert lse_rel_err(to64(lse[b, h]), l_ref) <= 1e-3, (b, h)


def test_fwd_fp8_workload(gpu_lib):
    B, H, N, d = 2, 32, 8192, 128
    seed = inputs.SEEDS["fp8_8k"]
    o, lse, (q, k, v) = fp8_case(gpu_lib, B, H, N, d, False, seed)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(seed)
    for b, h in [(0, 0), (1, 17), (1, 31)]:
        rows = _sample_rows(N, rng)
        o_ref, l_ref = oracle.attention_forward_rows(q[b, h], k[b, h], v[b, h], rows, d ** -0.5,
                                                     False)
        assert rel_frob(o[b, h, rows], o_ref) <= 5e-2, (b, h)
        assert lse_rel_err(lse[b, h, rows], l_ref) <= 1e-3, (b, h)


# ------------------------------------------------------------------ binding checks

def test_binding_rejects_mismatched_tensors(gpu_lib):
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.fa_fwd(q, q[:, :1].contiguous(), q, torch.empty_like(q), None, 0.1, False)
    with pytest.raises(TypeError):
        gpu_lib.fa_fwd(q, q.half(), q, torch.empty_like(q), None, 0.1, False)
    with pytest.raises(gpu_lib.FAError):
        x = torch.zeros(1, 2, 64, 96, dtype=torch.bfloat16, device="cuda")
        gpu_lib.fa_fwd(x, x, x, torch.empty_like(x), None, 0.1, False)


def test_max_size_fwd_bwd(gpu_lib):
    """B*H*N*d just below 2^31 (the ABI's limit): every index in the kernels
    crosses 2^30 elements. Inputs come from a seeded device generator (the
    host would need 26 GB); the first, a middle and the last head are checked
    against the oracle, the rest for finiteness."""
    B, H, N, d = 511, 32, 1024, 128
    assert B * H * N * d < 2 ** 31 and B * H * N * d > 2 ** 30 + 2 ** 29
    note(f"max size bf16 causal B{B} H{H} N{N} d{d}")
    g = torch.Generator(device="cuda")
    g.manual_seed(9001)
    shape = (B, H, N, d)
    q, k, v, do = (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
                   .to(torch.bfloat16) for _ in range(4))
    o, lse = gpu_lib.forward(q, k, v, causal=True)
    dq, dk, dv = gpu_lib.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    scale = d ** -0.5
    for b, h in ((0, 0), (B // 2, 17), (B - 1, H - 1)):
        args = [to64(t[b, h]) for t in (q, k, v)]
        o_ref, l_ref = oracle.attention_forward(*args, scale, True)
        assert max_abs(to64(o[b, h]), o_ref) <= 2e-2, (b, h)
        assert rel_frob(to64(o[b, h]), o_ref) <= 1e-2, (b, h)
        assert max_abs(to64(lse[b, h]), l_ref) <= 1e-3, (b, h)
        g_ref = oracle.attention_backward(*args, to64(do[b, h]), scale, True)
        for got, ref in zip((dq, dk, dv), g_ref):
            assert max_abs(to64(got[b, h]), ref) <= 5e-2, (b, h)
            assert rel_frob(to64(got[b, h]), ref) <= 1e-2, (b, h)
