"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Each source is compiled to its own object (in parallel, under _build/), then
the objects are linked into libfa.so. No source calls device code of another,
so no relocatable device code is needed.

build_all() also links libfa_serial.so, the race-guard build: the same sources
with FA_SERIAL_STAGING defined, so that every double-buffered kernel loads its
next LDS tile only after the current one is consumed. Its outputs must match
libfa.so bit for bit; it is a test build, not a product path.

Usage: python -m exact_io_aware_54_amd.build  (or call build_all()).
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
LIB_SERIAL = os.path.join(PKG, "libfa_serial.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_fwd_fp8.hip", "fa_bwd.hip",
           "fa_std.hip", "fa_splitkv.hip", "fa_v1.hip", "fa_convert.hip", "fa_probe.hip",
           "fa_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _compile(src, obj, extra_flags, verbose):
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + [
        "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, os.path.join(CSRC, src)]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose=False, extra_flags=(), out=LIB, jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]
    objs = [os.path.join(OBJDIR, f"{tag}.{os.path.splitext(s)[0]}.o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _compile(so[0], so[1], extra_flags, verbose),
                              zip(SOURCES, objs)))
    failed = [(s, r) for s, r in zip(SOURCES, results) if r.returncode != 0]
    for s, r in failed:
        sys.stderr.write(f"--- {s}\n{r.stdout}{r.stderr}")
    if failed:
        raise RuntimeError("hipcc failed building libfa.so: " + ", ".join(s for s, _ in failed))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libfa.so failed")
    os.replace(tmp, out)
    return out


def build_all(verbose=False, jobs=None):
    """libfa.so, then the race-guard build libfa_serial.so."""
    return [build(verbose=verbose, jobs=jobs),
            build(verbose=verbose, extra_flags=("-DFA_SERIAL_STAGING",), out=LIB_SERIAL,
                  jobs=jobs)]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
