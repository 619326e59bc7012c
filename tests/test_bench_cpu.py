"""CPU checks of bench.py's contract: one GPU only (a multi-GPU request exits
with a message before anything touches a device), the counted-FLOP
convention (4 B H N^2 d forward, half when causal, 2.5x for the backward),
and the command-line modes."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counted_flops_convention():
    b = load_bench()
    fwd = b.counted_flops(8, 16, 4096, 128, True)
    assert fwd == 4 * 8 * 16 * 4096 ** 2 * 128 / 2          # 549.8 GFLOP (C4 forward)
    assert abs(fwd - 549.755813888e9) < 1.0
    assert b.counted_flops(8, 16, 4096, 128, True, backward=True) == 2.5 * fwd
    assert b.counted_flops(2, 32, 8192, 128, False) == 4 * 2 * 32 * 8192 ** 2 * 128


def test_help_lists_modes():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--suite", "--fp8", "--tile-sweep", "--decode",
                 "--loop-order", "--compare-standard", "--calibrate-copy", "--sweep"):
        assert flag in r.stdout
