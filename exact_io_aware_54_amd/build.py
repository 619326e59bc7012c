"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m exact_io_aware_54_amd.build  (or call build()).
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_fwd_fp8.hip", "fa_bwd.hip",
           "fa_std.hip", "fa_splitkv.hip", "fa_v1.hip", "fa_convert.hip", "fa_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-x", "hip",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wno-unused-result",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False, extra_flags=()):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-I", os.path.join(ROOT, "include"),
                                                         "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
