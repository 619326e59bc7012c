"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic. It draws Q, K, V (and dO) from a
CPU ``torch.Generator`` as float32 N(0, 1), in the fixed order Q, K, V, dO, then
the outlier uniforms, and casts them on the CPU to the run dtype. The caller
moves them to the device; the oracle receives ``.double()`` of exactly the cast
(or dequantised) values.

The fp8 recipe: each element is multiplied by 20 with probability 0.01 (a
seeded uniform below 0.01), then the tensor is quantised to OCP E4M3 with the
per-tensor scale s = amax / 448 using torch's own float8_e4m3fn cast, after
clamping to +-448 (saturation). The kernels receive the E4M3 bytes and s as
the descale.
"""

import torch

# one seed per workload, as 1000 + workload index (ragged / long variants + 10)
SEEDS = {
    "tiny_f32": 1001,
    "fwd_bf16": 1002,
    "fwd_bf16_ragged": 1012,
    "causal_8k": 1003,
    "causal_16k": 1013,
    "train_4k": 1004,
    "fp8_8k": 1005,
    "decode_16k": 1021,   # split-KV parity: B4 H16 Nq1 Nk16384 d128
}

E4M3_MAX = 448.0


def draw_qkv(b, h, n, d, seed, dtype=torch.float32, with_do=False):
    """Return (q, k, v[, do]) CPU tensors [b, h, n, d] in ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (b, h, n, d)
    out = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3)]
    if with_do:
        out.append(torch.randn(shape, generator=g, dtype=torch.float32))
    return tuple(t.to(dtype).contiguous() for t in out)


def draw_qkv_rect(b, h, nq, nk, d, seed, dtype=torch.float32):
    """Return (q [b,h,nq,d], k [b,h,nk,d], v [b,h,nk,d]) CPU tensors in ``dtype``.

    Same recipe as draw_qkv (float32 N(0, 1), drawn in the order Q, K, V) with
    fewer queries than keys, for the split-KV (decoding) workloads.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((b, h, nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((b, h, nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((b, h, nk, d), generator=g, dtype=torch.float32)
    return tuple(t.to(dtype).contiguous() for t in (q, k, v))


def draw_qkv_rect_device(b, h, nq, nk, d, seed, dtype, device="cuda"):
    """Like draw_qkv_rect, but drawn by torch's generator on ``device``.

    For timing-only workloads too large to draw on the host (the values differ
    from the CPU draw of the same seed; parity tests use draw_qkv_rect).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((b, h, nq, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    k = torch.randn((b, h, nk, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    v = torch.randn((b, h, nk, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    return q, k, v


def draw_fp8(b, h, n, d, seed, outlier_p=0.01, outlier_mul=20.0):
    """Return ((q8, k8, v8) uint8 E4M3 codes, (sq, sk, sv) float descales).

    Draw order: Q, K, V normals, then one uniform tensor per input for the
    outlier selection.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (b, h, n, d)
    xs = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3)]
    us = [torch.rand(shape, generator=g, dtype=torch.float32) for _ in range(3)]
    codes, scales = [], []
    for x, u in zip(xs, us):
        x = torch.where(u < outlier_p, x * outlier_mul, x)
        s = (x.abs().max() / E4M3_MAX).to(torch.float32)
        xq = (x / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        codes.append(xq.view(torch.uint8).contiguous())
        scales.append(float(s))
    return tuple(codes), tuple(scales)
