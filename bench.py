#!/usr/bin/env python3
"""Benchmark: attention forward + backward TFLOPS on one MI355X.

Workload (one "step"): fa_fwd then the three launches of the backward
(fa_bwd_stage 1, 2, 3 = fa_bwd) on B=8, H=16, N=4096, d=128, bf16, causal,
with inputs already resident in HBM. Counted FLOPs: 4*B*H*N^2*d for the
forward, halved for causal, and 2.5x that for the backward.

The GPU's clocks ramp up over the first steps after the idle input
preparation (measured: the first step takes ~5 ms, steps settle at ~2.5 ms
after about 15 of them), so the default warm-up is 30 steps and the timed
region (50 steps) measures the steady state. The per-workload timings below
warm up for at least 60 ms of GPU work for the same reason.

Prints ONE JSON line on stdout. Besides the contract fields it carries
  roofline     -- for the kernel with the largest average duration, its
                  counted FLOPs / its HIP-event-timed duration against the
                  bf16 dense MFMA peak; traffic from the committed rocprofv3
                  PMC summary if it was taken on the current kernel source;
  cpu_baseline -- the float64 CPU oracle timed on a bounded sample of heads
                  of the same workload (reported, never a target);
  probe        -- the practical dense bf16 MFMA rate and the shader clock
                  under that load, from fa_probe_mfma (the measured ceiling
                  beside the spec peak);
  breakdown    -- per-launch times and TFLOPS.
`--suite PATH` additionally times every workload of the parity suite and
writes one JSON line per workload to PATH.
`--decode PATH` runs only the split-KV (few queries, many keys) workloads and
writes one JSON line per workload (median of 20 after the warm-up; HBM rate
from the bytes of Q, K, V and O read or written once).
`--loop-order PATH` runs only the loop-order ablation: the first-generation
order (fa_fwd_v1: K/V blocks outer, one workgroup per head, O / m / l through
memory) against the fused forward on the exercise shapes (B=1, H=32, d=128,
fp16, N = 2048 and 8192, causal and not; and B=8 at N=2048, where the
first-generation order has one workgroup per CU), one JSON line per case.
`--fp8 PATH` runs only the fp8 forward on its workload (B2 H32 N8192 d128,
causal and not), one JSON line per case.
`--bwd-design PATH` times the two-pass backward's launches on the training
workload against the dQ float atomics a one-pass backward would add
(fa_probe_dq_atomics), one JSON line per measurement.
`--sweep PATH` times the forward and the whole backward over sequence lengths
1K to 32K at the training workload's token count (bf16, d=128, H=16,
B = 32768 / N), causal and not, one JSON line per (N, causal, pass).
`--compare-standard PATH` runs only the comparison of the IO-aware forward with
the standard (materialising) forward that the pages' exercise describes
(B=1, H=32, d=128, fp16 random normals, N = 2048, 8192, 32768; at least 60 ms
of warm-up and 10 timed runs each; peak device memory from torch's allocator) and writes one
JSON line per sequence length to PATH.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
KERNEL_SOURCES = {
    "fwd_mfma_kernel": "exact_io_aware_54_amd/csrc/fa_fwd.hip",
    "bwd_dkdv_kernel": "exact_io_aware_54_amd/csrc/fa_bwd.hip",
    "bwd_dq_kernel": "exact_io_aware_54_amd/csrc/fa_bwd.hip",
    "fwd_fp8_dma_kernel": "exact_io_aware_54_amd/csrc/fa_fwd_fp8.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def counted_flops(B, H, N, d, causal, backward=False):
    f = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return 2.5 * f if backward else f


def source_sha(kernel):
    path = os.path.join(ROOT, KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "exact_io_aware_54_amd/csrc/fa_device.h")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed PMC summary, or None if stale/absent."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(q, k, v, do, scale, causal, budget_s, max_heads=96):
    """Time the float64 oracle on whole heads of the workload until budget_s is spent."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = 1
    B, H, N, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(heads))
    done, t0 = 0, time.perf_counter()
    for idx in order[:max_heads]:
        b, h = heads[idx]
        f64 = [t[b, h].float().numpy().astype(np.float64) for t in (q, k, v, do)]
        oracle.attention_forward(f64[0], f64[1], f64[2], scale, causal)
        oracle.attention_backward(f64[0], f64[1], f64[2], f64[3], scale, causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    flops = done * 3.5 * counted_flops(1, 1, N, d, causal)
    return {"value": flops / secs / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"fwd+bwd of {done} whole heads (N={N}, d={d}, causal) of the same "
                      f"workload in float64 numpy, {secs:.1f} s"}


def mfma_probe(torch, fa, blocks=512, iters=4096):
    """The practical dense bf16 MFMA rate and the shader clock under that load
    (fa_probe_mfma: 512 workgroups of four waves, two waves per SIMD, operands
    in registers). Returns None if the probe cannot run."""
    try:
        sink = torch.zeros(3 * blocks, device="cuda", dtype=torch.int64)
        run = lambda: fa.fa_probe_mfma(sink, blocks, iters)  # noqa: E731
        warm_up(run, torch, min_ms=20.0, min_calls=3)
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        flops = blocks * 4 * iters * 4 * 32768
        v = sink.view(blocks, 3).cpu().double()
        clk = sorted((v[:, 0] / v[:, 1]).tolist())[blocks // 2] * 100.0  # MHz
        return {"mfma_bf16_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                "sclk_mhz_under_mfma": round(clk, 0), "probe_ms": round(ms, 4),
                "note": "dense 32x32x16 bf16 MFMAs from registers; clock = s_memtime / "
                        "s_memrealtime ticks x 100 MHz (median over workgroups)"}
    except Exception as exc:  # a missing probe must not hide the bench line
        print(f"[bench] mfma probe failed: {exc}", file=sys.stderr, flush=True)
        return None


def warm_up(fn, torch, min_ms=60.0, min_calls=5):
    """Call `fn` until at least `min_calls` calls and `min_ms` of GPU time have run."""
    total, calls = 0.0, 0
    while calls < min_calls or total < min_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
        calls += 1
    return calls


def time_launches(fns, steps, warmup, torch):
    """Run `fns` in order per step; event-time each; return (wall_ms_per_step, [avg ms per fn])."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        evs[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            evs[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps
           for i in range(len(fns))]
    return wall, per


def calibration_copy(torch):
    """A plain device copy of known size (reads and writes exactly 1 GiB,
    three times): the HBM counters of a profiled run are scaled by what they
    read for it."""
    src = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_main(args):
    import torch
    import exact_io_aware_54_amd as fa
    from exact_io_aware_54_amd import inputs

    fa.load_library()
    if args.calibrate_copy:
        calibration_copy(torch)
    B, H, N, d, causal = 8, 16, 4096, 128, True
    scale = 1.0 / math.sqrt(d)
    print(f"[bench] drawing inputs B{B} H{H} N{N} d{d}", file=sys.stderr, flush=True)
    q, k, v, do = inputs.draw_qkv(B, H, N, d, inputs.SEEDS["train_4k"], torch.bfloat16, with_do=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = fa.workspace_for(qd)

    fns = [lambda: fa.fa_fwd(qd, kd, vd, o, lse, scale, causal)]
    for stage in (1, 2, 3):
        fns.append(lambda s=stage: fa.fa_bwd_stage(s, qd, kd, vd, o, lse, dod, dq, dk, dv, ws,
                                                   scale, causal))
    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall_ms, per = time_launches(fns, args.steps, args.warmup, torch)
    fwd_ms, pre_ms, main_ms, conv_ms = per  # stage 2 = dK/dV pass, stage 3 = dQ pass
    f_fwd = counted_flops(B, H, N, d, causal)
    f_bwd = counted_flops(B, H, N, d, causal, backward=True)
    value = (f_fwd + f_bwd) / (wall_ms * 1e-3) / 1e12
    bwd_ms = pre_ms + main_ms + conv_ms

    # Counted FLOPs per launch: the dK/dV pass does four of the backward's five
    # counted contractions (S, dP, dV, dK), the dQ pass recomputes S and dP and
    # adds dQ (three, of which only dQ is counted: 1/5 of the backward).
    cands = [("fwd_mfma_kernel", f_fwd, fwd_ms), ("bwd_dkdv_kernel", 0.8 * f_bwd, main_ms),
             ("bwd_dq_kernel", 0.2 * f_bwd, conv_ms)]
    kname, kflops, kms = max(cands, key=lambda t: t[2])
    achieved = kflops / (kms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(kname), "avg_launch_ms": round(kms, 4),
                "counted_flops_per_launch": kflops}

    probe = mfma_probe(torch, fa)
    if probe is not None:
        probe["value_frac_of_probe"] = round(value / probe["mfma_bf16_tflops"], 4)
        roofline["frac_of_probe"] = round(achieved / probe["mfma_bf16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(q, k, v, do, scale, causal, args.cpu_seconds)

    line = {
        "metric": "attention fwd+bwd TFLOPS (bf16, d=128, N=4K-16K) and % of MFMA peak, 1 GPU",
        "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fwd+bwd causal attention, B=8 H=16 N=4096 d=128 bf16",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "global_batch": B,
                   "seq_len": N, "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "probe": probe,
        "breakdown": {
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "bwd_stage_ms": {"pre": round(pre_ms, 4), "dkdv": round(main_ms, 4),
                             "dq": round(conv_ms, 4)},
            "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
            "fwd_frac_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_frac_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
    }
    print(json.dumps(line), flush=True)
    if args.suite:
        run_suite(args.suite, torch, fa, inputs)


def run_suite(path, torch, fa, inputs):
    """Median and minimum of 20 timed launches (after at least 60 ms of warm-up) for every workload."""
    import statistics
    cases = [
        ("fwd bf16 B4 H16 N2048 d64", "fwd", torch.bfloat16, 4, 16, 2048, 64, False, "fwd_bf16"),
        ("fwd bf16 B4 H16 N2000 d64 (ragged)", "fwd", torch.bfloat16, 4, 16, 2000, 64, False,
         "fwd_bf16_ragged"),
        ("fwd bf16 causal B1 H32 N8192 d128", "fwd", torch.bfloat16, 1, 32, 8192, 128, True,
         "causal_8k"),
        ("fwd bf16 causal B1 H32 N16384 d128", "fwd", torch.bfloat16, 1, 32, 16384, 128, True,
         "causal_16k"),
        ("fwd bf16 causal B8 H16 N4096 d128", "fwd", torch.bfloat16, 8, 16, 4096, 128, True,
         "train_4k"),
        ("fwd bf16 causal B1 H32 N8192 d256", "fwd", torch.bfloat16, 1, 32, 8192, 256, True,
         "causal_8k"),
        ("bwd bf16 causal B8 H16 N4096 d128", "bwd", torch.bfloat16, 8, 16, 4096, 128, True,
         "train_4k"),
        ("bwd bf16 causal B1 H32 N8192 d256", "bwd", torch.bfloat16, 1, 32, 8192, 256, True,
         "causal_8k"),
        ("fwd bf16 B1 H32 N8192 d256 (non-causal)", "fwd", torch.bfloat16, 1, 32, 8192, 256,
         False, "causal_8k"),
        ("bwd bf16 B1 H32 N8192 d256 (non-causal)", "bwd", torch.bfloat16, 1, 32, 8192, 256,
         False, "causal_8k"),
        ("fwd fp8 B2 H32 N8192 d128", "fp8", None, 2, 32, 8192, 128, False, "fp8_8k"),
        ("fwd fp8 causal B2 H32 N8192 d128", "fp8", None, 2, 32, 8192, 128, True, "fp8_8k"),
        # the fp8 backward widens the codes and runs the 16-bit passes: bf16 peak
        ("bwd fp8 B2 H32 N8192 d128", "fp8bwd", None, 2, 32, 8192, 128, False, "fp8_8k"),
        ("fwd f32 B1 H2 N128 d64", "fwd", torch.float32, 1, 2, 128, 64, False, "tiny_f32"),
        ("fwd f32 B4 H16 N2048 d64", "fwd", torch.float32, 4, 16, 2048, 64, False, "fwd_bf16"),
        ("fwd f32 causal B1 H32 N4096 d128", "fwd", torch.float32, 1, 32, 4096, 128, True,
         "causal_8k"),
    ]
    out = open(path, "w")
    for name, kind, dt, B, H, N, d, causal, seedkey in cases:
        print(f"[suite] {name}", file=sys.stderr, flush=True)
        scale = d ** -0.5
        seed = inputs.SEEDS[seedkey]
        if kind == "fp8":
            (q8, k8, v8), sc = inputs.draw_fp8(B, H, N, d, seed)
            q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
            o = torch.empty((B, H, N, d), device="cuda", dtype=torch.bfloat16)
            lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
            fn = lambda: fa.fa_fwd_fp8(q8, k8, v8, sc[0], sc[1], sc[2], o, lse, scale, causal)  # noqa
            flops, peak = counted_flops(B, H, N, d, causal), PEAK_FP8_TFLOPS
        elif kind == "fp8bwd":
            (q8, k8, v8), sc = inputs.draw_fp8(B, H, N, d, seed)
            q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
            o, lse = fa.forward_fp8(q8, k8, v8, sc, scale=scale, causal=causal)
            g = torch.Generator().manual_seed(seed + 1)
            do = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).cuda()
            dq, dk, dv = (torch.empty((B, H, N, d), device="cuda", dtype=torch.bfloat16)
                          for _ in range(3))
            ws = torch.empty(fa.fa_bwd_fp8_workspace_bytes(B, H, N, d), device="cuda",
                             dtype=torch.uint8)
            fn = lambda: fa.fa_bwd_fp8(q8, k8, v8, sc[0], sc[1], sc[2], o, lse, do, dq, dk, dv,  # noqa
                                       ws, scale, causal)
            flops, peak = counted_flops(B, H, N, d, causal, backward=True), PEAK_BF16_TFLOPS
        else:
            q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, dt, with_do=True))
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
            fa.fa_fwd(q, k, v, o, lse, scale, causal)
            if kind == "fwd":
                fn = lambda: fa.fa_fwd(q, k, v, o, lse, scale, causal)  # noqa
                flops = counted_flops(B, H, N, d, causal)
            else:
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                ws = fa.workspace_for(q)
                fn = lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal)  # noqa
                flops = counted_flops(B, H, N, d, causal, backward=True)
            peak = PEAK_FP32_TFLOPS if dt == torch.float32 else PEAK_BF16_TFLOPS
        warm_up(fn, torch)
        times = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        med, mn = statistics.median(times), min(times)
        rec = {"workload": name, "median_ms": round(med, 4), "min_ms": round(mn, 4),
               "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
               "frac_peak_median": round(flops / (med * 1e-3) / 1e12 / peak, 4), "seed": seed}
        print(json.dumps(rec), file=out, flush=True)
        print(f"[suite] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del fn
        torch.cuda.empty_cache()
    out.close()


def run_sweep(path, torch, fa, inputs, lengths=(1024, 2048, 4096, 8192, 16384, 32768)):
    """Sequence-length sweep at a fixed token count: bf16, d = 128, H = 16, B = 32768 / N
    (the training workload's B*N), causal and not. The forward and the whole backward
    (fa_bwd: row terms, dK/dV pass, dQ pass), medians of 20 HIP-event-timed calls after
    at least 60 ms of warm-up each, one JSON line per (N, causal, pass)."""
    import statistics
    H, d = 16, 128
    scale = d ** -0.5
    out = open(path, "w")
    for N in lengths:
        B = max(1, 32768 // N)
        q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, inputs.SEEDS["train_4k"],
                                                          torch.bfloat16, with_do=True))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = fa.workspace_for(q)
        for causal in (True, False):
            fa.fa_fwd(q, k, v, o, lse, scale, causal)
            passes = (("fwd", lambda: fa.fa_fwd(q, k, v, o, lse, scale, causal)),  # noqa
                      ("bwd", lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale,  # noqa
                                                causal)))
            for pname, fn in passes:
                print(f"[sweep] N{N} B{B} causal={causal} {pname}", file=sys.stderr, flush=True)
                warm_up(fn, torch)
                times = []
                for _ in range(20):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1))
                med = statistics.median(times)
                flops = counted_flops(B, H, N, d, causal, backward=(pname == "bwd"))
                tf = flops / (med * 1e-3) / 1e12
                rec = {"pass": pname, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                       "median_ms": round(med, 4), "tflops": round(tf, 1),
                       "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
                print(json.dumps(rec), file=out, flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    out.close()


def run_compare(path, torch, fa, inputs, lengths=(2048, 8192, 32768)):
    """IO-aware forward vs standard forward: time and peak memory per length."""
    B, H, d = 1, 32, 128
    scale = d ** -0.5
    out = open(path, "w")
    for N in lengths:
        seed = 1100 + N // 1024
        print(f"[compare] N={N} seed={seed}", file=sys.stderr, flush=True)
        q, k, v = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, torch.float16))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        rec = {"workload": f"fwd f16 B{B} H{H} N{N} d{d} non-causal", "seed": seed}
        for name in ("flash", "standard"):
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            o = torch.empty_like(q)
            if name == "flash":
                lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
                fn = lambda: fa.fa_fwd(q, k, v, o, lse, scale, False)  # noqa: E731
            else:
                ws = torch.empty(fa.fa_std_workspace_bytes(B, H, N, d), device="cuda",
                                 dtype=torch.uint8)
                fn = lambda: fa.fa_std_fwd(q, k, v, o, ws, scale, False)  # noqa: E731
            warm_up(fn, torch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            peak = torch.cuda.max_memory_allocated()
            rec[name] = {"time_ms": round(ms, 3),
                         "tflops": round(counted_flops(B, H, N, d, False) / (ms * 1e-3) / 1e12, 1),
                         "peak_mib": round(peak / 2 ** 20, 1),
                         "beyond_inputs_mib": round((peak - base) / 2 ** 20, 1)}
            print(f"[compare]   {name}: {rec[name]}", file=sys.stderr, flush=True)
            del fn, o
            if name == "flash":
                del lse
            else:
                del ws
        rec["speedup"] = round(rec["standard"]["time_ms"] / rec["flash"]["time_ms"], 2)
        rec["memory_ratio_beyond_inputs"] = round(
            rec["standard"]["beyond_inputs_mib"] / rec["flash"]["beyond_inputs_mib"], 1)
        print(json.dumps(rec), file=out, flush=True)
        print(f"[compare] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del q, k, v
        torch.cuda.empty_cache()
    out.close()


DECODE_CASES = [
    # (name, B, H, Nq, Nk, d, causal, seed)
    ("decode bf16 B8 H32 Nq1 Nk32768 d128", 8, 32, 1, 32768, 128, False, 1031),
    ("decode bf16 B1 H32 Nq1 Nk131072 d128", 1, 32, 1, 131072, 128, False, 1032),
    ("chunk bf16 causal B8 H32 Nq16 Nk8192 d128", 8, 32, 16, 8192, 128, True, 1033),
]


def run_decode(path, torch, fa, inputs):
    """Split-KV forward on decoding-shaped workloads: time and HBM rate."""
    import statistics
    out = open(path, "w")
    for name, B, H, Nq, Nk, d, causal, seed in DECODE_CASES:
        print(f"[decode] {name}", file=sys.stderr, flush=True)
        q, k, v = inputs.draw_qkv_rect_device(B, H, Nq, Nk, d, seed, torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), device="cuda", dtype=torch.float32)
        ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0), device="cuda",
                         dtype=torch.uint8)
        fn = lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, ws, d ** -0.5, causal, 0)  # noqa: E731
        warm_up(fn, torch)
        times = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        med = statistics.median(times)
        nbytes = 2 * (2 * B * H * Nq * d + 2 * B * H * Nk * d) + 4 * B * H * Nq
        rec = {"workload": name, "median_ms": round(med, 4), "min_ms": round(min(times), 4),
               "hbm_gbs": round(nbytes / (med * 1e-3) / 1e9, 1),
               "frac_hbm": round(nbytes / (med * 1e-3) / 8.0e12, 4),
               "algorithmic_bytes": nbytes, "seed": seed}
        print(json.dumps(rec), file=out, flush=True)
        print(f"[decode] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del q, k, v, o, lse, ws, fn
        torch.cuda.empty_cache()
    out.close()


def run_loop_order(path, torch, fa, inputs):
    """First-generation loop order vs the fused (second-generation) forward."""
    H, d = 32, 128
    scale = d ** -0.5
    out = open(path, "w")
    # B = 8 gives the first-generation order one workgroup per CU (256 heads), so
    # its gap to the fused kernel there is the loop order and round trips alone
    for B, N, causal in ((1, 2048, False), (1, 2048, True), (1, 8192, False), (1, 8192, True),
                         (8, 2048, False)):
        seed = 1100 + N // 1024 + (B - 1)
        print(f"[loop-order] N={N} causal={causal}", file=sys.stderr, flush=True)
        q, k, v = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, torch.float16))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
        ws = torch.empty(fa.fa_fwd_v1_workspace_bytes(B, H, N, d), device="cuda",
                         dtype=torch.uint8)
        fns = {"v1_kv_outer": lambda: fa.fa_fwd_v1(q, k, v, o, lse, ws, scale, causal),
               "v2_fused": lambda: fa.fa_fwd(q, k, v, o, lse, scale, causal)}
        rec = {"workload": f"fwd f16 B{B} H{H} N{N} d{d} causal={causal}", "seed": seed}
        flops = counted_flops(B, H, N, d, causal)
        for name, fn in fns.items():
            reps = 3 if name == "v1_kv_outer" else 10
            warm_up(fn, torch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            rec[name] = {"time_ms": round(ms, 3),
                         "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        # O, m, l round trips of the first-generation order: per (K/V block of 64,
        # Q block of 128) pair, O (fp32) and Q are read and O written
        nkb, nqb = (N + 63) // 64, (N + 127) // 128
        pairs = nkb * nqb if not causal else sum(
            1 for j in range(nkb) for i in range(nqb) if j * 64 <= i * 128 + 127)
        rec["v1_round_trip_bytes"] = B * H * pairs * 128 * d * (4 + 4 + 2)
        rec["speedup_v2_over_v1"] = round(rec["v1_kv_outer"]["time_ms"] /
                                          rec["v2_fused"]["time_ms"], 1)
        print(json.dumps(rec), file=out, flush=True)
        print(f"[loop-order] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del q, k, v, o, lse, ws, fns
        torch.cuda.empty_cache()
    out.close()


def run_tile_sweep(path, torch, fa, inputs, calibrate=False):
    """The forward's two workgroup shapes (four and eight waves) on each bf16
    forward workload, medians of 20 event-timed launches after the warm-up."""
    if calibrate:
        calibration_copy(torch)
    cases = [("C2", 4, 16, 2048, 64, False, 1002), ("C3a", 1, 32, 8192, 128, True, 1003),
             ("C3b", 1, 32, 16384, 128, True, 1013), ("C4", 8, 16, 4096, 128, True, 1004),
             ("non-causal", 2, 32, 8192, 128, False, 1005)]
    out = open(path, "w")
    for name, B, H, N, d, causal, seed in cases:
        print(f"[tile-sweep] {name} B{B} H{H} N{N} d{d} causal={causal}", file=sys.stderr,
              flush=True)
        q, k, v = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, torch.bfloat16))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
        flops = counted_flops(B, H, N, d, causal)
        rec = {"workload": f"fwd bf16 {name} B{B} H{H} N{N} d{d} causal={causal}", "seed": seed,
               "default_waves": 8 if B * H * ((N + 255) // 256) >= 256 else 4}
        for waves in (4, 8):
            fn = lambda: fa.fa_fwd_waves(q, k, v, o, lse, d ** -0.5, causal, waves)
            warm_up(fn, torch)
            times = []
            for _ in range(20):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            med = sorted(times)[len(times) // 2]
            rec[f"waves{waves}"] = {"median_ms": round(med, 4),
                                    "tflops": round(flops / (med * 1e-3) / 1e12, 1)}
        print(json.dumps(rec), file=out, flush=True)
        print(f"[tile-sweep] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    out.close()


def _median_ms(fn, torch, n=20):
    warm_up(fn, torch)
    times = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return sorted(times)[len(times) // 2]


def run_bwd_design(path, torch, fa, inputs):
    """The backward's structure, measured on the causal B8 H16 N4096 d128
    workload: the two-pass backward's three launches (row terms, dK/dV, dQ)
    against the float atomics a one-pass backward would add to its dK/dV pass
    (fa_probe_dq_atomics: the same stream of dQ partial additions with no
    arithmetic around it, for 128- and 256-key blocks, and plain stores of the
    same addresses). Medians of 20 event-timed launches after the warm-up, one
    JSON line per measurement and a summary line."""
    B, H, N, d, causal = 8, 16, 4096, 128, True
    scale = d ** -0.5
    q, k, v, do = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, inputs.SEEDS["train_4k"],
                                                      torch.bfloat16, with_do=True))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    fa.fa_fwd(q, k, v, o, lse, scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = fa.workspace_for(q)
    out = open(path, "w")
    rec = {"design": "two-pass", "workload": f"bwd bf16 causal B{B} H{H} N{N} d{d}"}
    for stage, name in ((1, "pre"), (2, "dkdv"), (3, "dq")):
        fn = lambda s=stage: fa.fa_bwd_stage(s, q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal)  # noqa
        rec[f"{name}_ms"] = round(_median_ms(fn, torch), 4)
    rec["bwd_ms"] = round(rec["pre_ms"] + rec["dkdv_ms"] + rec["dq_ms"], 4)
    print(json.dumps(rec), file=out, flush=True)
    print(f"[bwd-design] {json.dumps(rec)}", file=sys.stderr, flush=True)
    acc = torch.zeros(B * H * N * 128, device="cuda", dtype=torch.float32)
    probes = {}
    for kb in (128, 256):
        pairs = sum(N // 64 - (j * kb) // 64 for j in range(N // kb))
        nbytes = B * H * pairs * 64 * 128 * 4
        for mode, mname in ((0, "atomic_add"), (1, "plain_store")):
            fn = lambda kb=kb, m=mode: fa.fa_probe_dq_atomics(acc, B, H, N, kb, m, causal)  # noqa
            ms = _median_ms(fn, torch)
            probes[(kb, mname)] = ms
            r = {"design": "one-pass dQ traffic alone", "key_block": kb, "op": mname,
                 "median_ms": round(ms, 4), "bytes": nbytes,
                 "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            print(json.dumps(r), file=out, flush=True)
            print(f"[bwd-design] {json.dumps(r)}", file=sys.stderr, flush=True)
    summ = {"summary": "a one-pass backward takes at least its dQ atomics' time; the two-pass "
                       "backward's dQ pass is the time it would save",
            "two_pass_bwd_ms": rec["bwd_ms"], "two_pass_dq_pass_ms": rec["dq_ms"],
            "one_pass_atomics_ms_kb128": round(probes[(128, "atomic_add")], 4),
            "one_pass_atomics_ms_kb256": round(probes[(256, "atomic_add")], 4)}
    print(json.dumps(summ), file=out, flush=True)
    print(f"[bwd-design] {json.dumps(summ)}", file=sys.stderr, flush=True)
    out.close()


def run_fp8(path, torch, fa, inputs, calibrate=False):
    """The fp8 forward alone on C5's shape (B2 H32 N8192 d128, E4M3 with 1 %
    x20 outliers), non-causal (the graded case) and causal: medians of 20
    event-timed launches after at least 60 ms of warm-up, one JSON line each."""
    if calibrate:
        calibration_copy(torch)
    B, H, N, d = 2, 32, 8192, 128
    seed = inputs.SEEDS["fp8_8k"]
    (q8, k8, v8), sc = inputs.draw_fp8(B, H, N, d, seed)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    o = torch.empty((B, H, N, d), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    out = open(path, "w")
    for causal in (False, True):
        fn = lambda: fa.fa_fwd_fp8(q8, k8, v8, sc[0], sc[1], sc[2], o, lse, d ** -0.5, causal)  # noqa
        warm_up(fn, torch)
        times = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        med = sorted(times)[len(times) // 2]
        flops = counted_flops(B, H, N, d, causal)
        rec = {"workload": f"fwd fp8 e4m3 B{B} H{H} N{N} d{d} causal={causal}", "seed": seed,
               "median_ms": round(med, 4), "tflops": round(flops / (med * 1e-3) / 1e12, 1),
               "frac_fp8_peak": round(flops / (med * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        print(json.dumps(rec), file=out, flush=True)
        print(f"[fp8] {json.dumps(rec)}", file=sys.stderr, flush=True)
    out.close()


F32_CASES = [
    # (name, B, H, N, d, causal, seed key)
    ("fwd f32 B1 H2 N128 d64", 1, 2, 128, 64, False, "tiny_f32"),
    ("fwd f32 B4 H16 N2048 d64", 4, 16, 2048, 64, False, "fwd_bf16"),
    ("fwd f32 causal B1 H32 N4096 d128", 1, 32, 4096, 128, True, "causal_8k"),
    ("fwd f32 B1 H32 N4096 d128", 1, 32, 4096, 128, False, "causal_8k"),
]


def run_f32(path, torch, fa, inputs, calibrate=False):
    """The fp32 forward alone: the tiny parity workload and longer shapes,
    medians of 20 event-timed launches after at least 60 ms of warm-up, one
    JSON line each, against the fp32 MFMA peak."""
    if calibrate:
        calibration_copy(torch)
    out = open(path, "w")
    for name, B, H, N, d, causal, seedkey in F32_CASES:
        seed = inputs.SEEDS[seedkey]
        q, k, v = (t.cuda() for t in inputs.draw_qkv(B, H, N, d, seed, torch.float32))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
        fn = lambda: fa.fa_fwd(q, k, v, o, lse, d ** -0.5, causal)  # noqa: E731
        warm_up(fn, torch)
        times = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        med = sorted(times)[len(times) // 2]
        flops = counted_flops(B, H, N, d, causal)
        rec = {"workload": name, "seed": seed, "median_ms": round(med, 4),
               "tflops": round(flops / (med * 1e-3) / 1e12, 2),
               "frac_fp32_peak": round(flops / (med * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
        print(json.dumps(rec), file=out, flush=True)
        print(f"[f32] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del q, k, v, o, lse, fn
        torch.cuda.empty_cache()
    out.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", metavar="PATH", help="also time every workload, JSON lines to PATH")
    ap.add_argument("--loop-order", metavar="PATH",
                    help="only run the loop-order ablation, JSON lines to PATH")
    ap.add_argument("--decode", metavar="PATH",
                    help="only run the split-KV decoding workloads, JSON lines to PATH")
    ap.add_argument("--compare-standard", metavar="PATH",
                    help="only run the IO-aware vs standard forward comparison, JSON lines to PATH")
    ap.add_argument("--compare-n", type=int, nargs="+", default=[2048, 8192, 32768],
                    help="sequence lengths of --compare-standard")
    ap.add_argument("--tile-sweep", metavar="PATH",
                    help="only time the forward's four- and eight-wave workgroup shapes on each "
                         "bf16 forward workload, JSON lines to PATH")
    ap.add_argument("--f32", metavar="PATH",
                    help="only time the fp32 forward (tiny and longer shapes), JSON lines to PATH")
    ap.add_argument("--fp8", metavar="PATH",
                    help="only time the fp8 forward on its workload (causal and not), JSON lines "
                         "to PATH")
    ap.add_argument("--bwd-design", metavar="PATH",
                    help="only time the two-pass backward's launches against the dQ float "
                         "atomics a one-pass backward would add, JSON lines to PATH")
    ap.add_argument("--sweep", metavar="PATH",
                    help="only run the sequence-length sweep (bf16 d128, B*N = 32768, forward "
                         "and backward, causal and not), JSON lines to PATH")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy, the reference kernel for scaling "
                         "PMC byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: attention shards by (batch, head) with no "
              "communication, so the whole-job rate at N GPUs is N times the 1-GPU figure at "
              "the per-GPU head count; run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    if (args.decode or args.compare_standard or args.loop_order or args.tile_sweep or args.fp8
            or args.bwd_design or args.f32 or args.sweep):
        import torch
        import exact_io_aware_54_amd as fa
        from exact_io_aware_54_amd import inputs
        if not torch.cuda.is_available():
            sys.exit("bench.py needs a GPU")
        fa.load_library()
        if args.decode:
            run_decode(args.decode, torch, fa, inputs)
        if args.loop_order:
            run_loop_order(args.loop_order, torch, fa, inputs)
        if args.tile_sweep:
            run_tile_sweep(args.tile_sweep, torch, fa, inputs, args.calibrate_copy)
        if args.compare_standard:
            run_compare(args.compare_standard, torch, fa, inputs, args.compare_n)
        if args.fp8:
            run_fp8(args.fp8, torch, fa, inputs, args.calibrate_copy)
        if args.f32:
            run_f32(args.f32, torch, fa, inputs, args.calibrate_copy)
        if args.bwd_design:
            run_bwd_design(args.bwd_design, torch, fa, inputs)
        if args.sweep:
            run_sweep(args.sweep, torch, fa, inputs)
        return
    run_main(args)


if __name__ == "__main__":
    main()
