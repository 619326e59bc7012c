"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

csrc/fa_api.cpp (argument validation, workspace carving, dispatch) is built
with g++ -fsanitize=address,undefined together with host-only stand-ins for
the kernel launchers and the three HIP runtime calls it makes
(tests/host/fa_host_stubs.cpp), and driven by tests/host/fa_host_check.cpp:
every entry point with valid and invalid arguments, the launch arguments of
valid calls (every sub-buffer carved from a workspace lies inside the size
the matching *_workspace_bytes function reports, without overlaps), the
error state around launches, and a sweep of extreme sizes (INT_MIN to
INT_MAX) for overflow in the size arithmetic. No kernel and no GPU is
involved: the launchers only record their arguments.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "exact_io_aware_54_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "tests", "host", "fa_host_stubs.cpp"),
           os.path.join(ROOT, "tests", "host", "fa_host_check.cpp")]


def test_abi_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "fa_host_check")
    build = subprocess.run(
        [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-o", exe] + SOURCES, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert " 0 failed" in run.stdout, run.stdout
