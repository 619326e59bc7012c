"""Host-side checks of libfa's C ABI (CPU only, no kernel is ever launched).

The library must load and export every function declared in include/fa.h.
Invalid arguments must be rejected with the documented status before any HIP
call, so these calls are safe without a GPU: every call below is invalid.
"""

import ctypes
import os
import re

import pytest

import exact_io_aware_54_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_io_aware_54_amd import build
        build.build()
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_bwd_stage",
                          "fa_bwd_workspace_bytes", "fa_status_string", "fa_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in list(fa.STATUS) + [-99]:
        s = fa.fa_status_string(code)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(0) == "ok"
    assert fa.fa_version() >= 100


def test_workspace_bytes(lib):
    B, H, N, d = 2, 3, 100, 64
    rows = B * H * N
    want = 2 * (-(-rows * 4 // 256) * 256)
    assert fa.fa_bwd_workspace_bytes(B, H, N, d) == want
    assert fa.fa_bwd_workspace_bytes(0, H, N, d) == 0
    assert fa.fa_bwd_workspace_bytes(B, H, N, 96) == 0


def fwd(lib, **kw):
    a = dict(dtype=fa.FA_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0)
    a.update(kw)
    return lib.fa_fwd(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                      a["N"], a["d"], a["scale"], a["causal"], None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == -1
    assert fwd(lib, o=None) == -1
    assert fwd(lib, dtype=7) == -3
    assert fwd(lib, B=0) == -2
    assert fwd(lib, N=-5) == -2
    assert fwd(lib, d=96) == -4
    assert fwd(lib, d=512) == -4
    assert fwd(lib, dtype=fa.FA_F32, d=256) == -4   # 256 only on the 16-bit path
    assert fwd(lib, d=256, B=1 << 14, H=1 << 10, N=1 << 10) == -2
    assert fwd(lib, B=1 << 14, H=1 << 10, N=1 << 10, d=128) == -2  # 2^41 elements
    assert fwd(lib, scale=0.0) == -7
    assert fwd(lib, scale=float("nan")) == -7
    assert fwd(lib, scale=float("inf")) == -7


def test_fp8_validation(lib):
    def f8(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sq=1.0, sk=1.0, sv=1.0, o=FAKE, d=128, scale=0.1)
        a.update(kw)
        return lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["sq"], a["sk"], a["sv"], a["o"], FAKE,
                              1, 1, 64, a["d"], a["scale"], 0, None)
    assert f8(v=None) == -1
    assert f8(d=64) == -4
    assert f8(sq=0.0) == -7
    assert f8(sv=-1.0) == -7
    assert f8(sk=float("nan")) == -7
    assert f8(scale=-0.5) == -7


def test_bwd_validation(lib):
    B, H, N, d = 1, 2, 64, 64
    need = fa.fa_bwd_workspace_bytes(B, H, N, d)

    def bwd(stage=None, **kw):
        a = dict(dtype=fa.FA_BF16, ws=ctypes.c_void_p(0x10000), wsb=need, d=d, scale=0.1, do=FAKE)
        a.update(kw)
        args = [a["dtype"], FAKE, FAKE, FAKE, FAKE, FAKE, a["do"], FAKE, FAKE, FAKE, a["ws"],
                a["wsb"], B, H, N, a["d"], a["scale"], 1, None]
        if stage is None:
            return lib.fa_bwd(*args)
        return lib.fa_bwd_stage(stage, *args)

    assert bwd(do=None) == -1
    assert bwd(ws=None) == -1
    assert bwd(dtype=fa.FA_F32) == -3
    assert bwd(d=80) == -4
    assert bwd(d=512) == -4
    assert bwd(wsb=need - 1) == -5
    assert bwd(ws=ctypes.c_void_p(0x10010)) == -5  # not 256-byte aligned
    assert bwd(scale=0.0) == -7
    assert bwd(stage=0) == -7
    assert bwd(stage=4) == -7
    assert bwd(stage=2, wsb=0) == -5


def test_std_workspace_bytes(lib):
    # one 16-bit N x N score matrix per (batch, head)
    assert fa.fa_std_workspace_bytes(2, 3, 100, 64) == 2 * 3 * 100 * 100 * 2
    assert fa.fa_std_workspace_bytes(1, 32, 32768, 128) == 32 * 32768 * 32768 * 2  # > 2^32
    assert fa.fa_std_workspace_bytes(0, 1, 16, 64) == 0
    assert fa.fa_std_workspace_bytes(1, 1, 16, 96) == 0


def test_std_validation(lib):
    B, H, N, d = 1, 2, 64, 64
    need = fa.fa_std_workspace_bytes(B, H, N, d)

    def std(**kw):
        a = dict(dtype=fa.FA_BF16, q=FAKE, ws=ctypes.c_void_p(0x10000), wsb=need, B=B, H=H,
                 d=d, scale=0.1)
        a.update(kw)
        return lib.fa_std_fwd(a["dtype"], a["q"], FAKE, FAKE, FAKE, a["ws"], a["wsb"], a["B"],
                              a["H"], N, a["d"], a["scale"], 0, None)

    assert std(q=None) == -1
    assert std(ws=None) == -1
    assert std(dtype=fa.FA_F32) == -3
    assert std(dtype=7) == -3
    assert std(d=32) == -4
    assert std(B=0) == -2
    assert std(B=256, H=256) == -2  # B*H beyond the score pass's grid limit
    assert std(wsb=need - 1) == -5
    assert std(ws=ctypes.c_void_p(0x10010)) == -5
    assert std(scale=float("inf")) == -7


def test_library_has_no_unresolved_kernel_stubs():
    # A kernel whose host-side launch stub was not emitted shows up as an
    # undefined __device_stub__ symbol and makes dlopen fail on first use.
    import subprocess
    for path in (fa.LIB_PATH, fa.SERIAL_LIB_PATH):
        if not os.path.exists(path):
            continue
        out = subprocess.run(["nm", "-D", path], capture_output=True, text=True).stdout
        missing = [ln for ln in out.splitlines() if " U " in ln and "__device_stub__" in ln]
        assert missing == [], path


def test_race_guard_build_flags(lib):
    # The product library reports no build variant; the race-guard build
    # (serial LDS staging) loads, exports the same symbols and says what it is.
    assert fa.fa_build_flags() == 0
    if not os.path.exists(fa.SERIAL_LIB_PATH):
        from exact_io_aware_54_amd import build
        build.build_all()
    serial = ctypes.CDLL(fa.SERIAL_LIB_PATH)
    for n in declared_functions():
        assert hasattr(serial, n), n
    serial.fa_build_flags.restype = ctypes.c_int
    assert serial.fa_build_flags() == 1
    with fa.library_override(fa.SERIAL_LIB_PATH):
        assert fa.fa_build_flags() == 1
        # validation is shared: an invalid call is rejected the same way
        assert fa.load_library().fa_fwd(2, None, FAKE, FAKE, FAKE, None, 1, 1, 64, 64,
                                        0.125, 0, None) == -1
    assert fa.fa_build_flags() == 0


def test_splitkv_workspace_bytes(lib):
    # 8 tiles of 128 keys, 4 requested ranges -> 4 ranges of 2 tiles;
    # partial O: 4 * (1*2*3) rows * 64 floats, partial LSE: 24 floats (each padded to 256 B)
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 1000, 64, 4) == 6144 + 256
    # automatic: 2 (batch*head*query-block) units -> 256 wanted, capped at the 8 tiles
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 1000, 64, 0) == 12288 + 256
    # 7 requested of 8 tiles -> 2 tiles per range -> 4 ranges
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 1000, 64, 7) == 6144 + 256
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 1000, 80, 1) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 1000, 64, -1) == 0


def test_splitkv_validation(lib):
    B, H, Nq, Nk, d = 1, 2, 4, 300, 64
    need = fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 2)

    def skv(**kw):
        a = dict(dtype=fa.FA_BF16, q=FAKE, Nq=Nq, Nk=Nk, d=d, scale=0.1, causal=0, ns=2,
                 ws=ctypes.c_void_p(0x10000), wsb=need)
        a.update(kw)
        return lib.fa_fwd_splitkv(a["dtype"], a["q"], FAKE, FAKE, FAKE, None, B, H, a["Nq"],
                                  a["Nk"], a["d"], a["scale"], a["causal"], a["ns"], a["ws"],
                                  a["wsb"], None)

    assert skv(q=None) == -1
    assert skv(ws=None) == -1
    assert skv(dtype=fa.FA_F32) == -3
    assert skv(d=96) == -4
    assert skv(Nq=0) == -2
    assert skv(Nk=0) == -2
    assert skv(causal=1, Nq=400) == -2       # causal needs Nq <= Nk
    assert skv(ns=-1) == -7
    assert skv(ns=1025) == -7
    assert skv(scale=-1.0) == -7
    assert skv(wsb=need - 1) == -5
    assert skv(ws=ctypes.c_void_p(0x10008)) == -5


def test_lse_merge_validation(lib):
    def merge(**kw):
        a = dict(dt=fa.FA_F32, P=2, op=ctypes.c_void_p(0x10000), lp=FAKE, o=FAKE, rows=10, d=64)
        a.update(kw)
        return lib.fa_lse_merge(a["dt"], a["P"], a["op"], a["lp"], a["o"], None, a["rows"],
                                a["d"], None)

    assert merge(op=None) == -1
    assert merge(lp=None) == -1
    assert merge(o=None) == -1
    assert merge(dt=9) == -3
    assert merge(P=0) == -2
    assert merge(rows=0) == -2
    assert merge(d=6) == -2
    assert merge(d=0) == -2
    assert merge(op=ctypes.c_void_p(0x10004)) == -7  # o_parts not 16-byte aligned


def test_v1_workspace_and_validation(lib):
    B, H, N, d = 1, 2, 100, 64
    rows = B * H * N
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    need = fa.fa_fwd_v1_workspace_bytes(B, H, N, d)
    assert need == a256(rows * d * 4) + 2 * a256(rows * 2 * 4)
    assert fa.fa_fwd_v1_workspace_bytes(B, H, N, 256) == 0

    def v1(**kw):
        a = dict(dtype=fa.FA_BF16, q=FAKE, ws=ctypes.c_void_p(0x10000), wsb=need, d=d, scale=0.1)
        a.update(kw)
        return lib.fa_fwd_v1(a["dtype"], a["q"], FAKE, FAKE, FAKE, None, a["ws"], a["wsb"], B, H,
                             N, a["d"], a["scale"], 0, None)

    assert v1(q=None) == -1
    assert v1(ws=None) == -1
    assert v1(dtype=fa.FA_F32) == -3
    assert v1(d=256) == -4
    assert v1(scale=0.0) == -7
    assert v1(wsb=need - 1) == -5
    assert v1(ws=ctypes.c_void_p(0x10040)) == -5


def test_misaligned_pointers_rejected(lib):
    odd = ctypes.c_void_p(0x1008)   # 8-byte but not 16-byte aligned
    assert fwd(lib, q=odd) == -7
    assert fwd(lib, o=odd) == -7
    assert fwd(lib, lse=ctypes.c_void_p(0x1002)) == -7
    assert lib.fa_fwd_fp8(odd, FAKE, FAKE, 1.0, 1.0, 1.0, FAKE, FAKE, 1, 1, 64, 128, 0.1, 0,
                          None) == -7
    need = fa.fa_bwd_workspace_bytes(1, 1, 64, 64)
    assert lib.fa_bwd(fa.FA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, odd, FAKE,
                      ctypes.c_void_p(0x10000), need, 1, 1, 64, 64, 0.1, 0, None) == -7


def test_bwd_fp8_workspace_bytes(lib):
    B, H, N, d = 1, 2, 100, 128
    codes = -(-B * H * N * d * 2 // 256) * 256          # one bf16 copy, padded to 256 B
    assert fa.fa_bwd_fp8_workspace_bytes(B, H, N, d) == 3 * codes + \
        fa.fa_bwd_workspace_bytes(B, H, N, d)
    assert fa.fa_bwd_fp8_workspace_bytes(B, H, N, 96) == 0
    assert fa.fa_bwd_fp8_workspace_bytes(0, H, N, d) == 0


def test_bwd_fp8_validation(lib):
    B, H, N, d = 1, 2, 64, 128
    need = fa.fa_bwd_fp8_workspace_bytes(B, H, N, d)

    def f8b(**kw):
        a = dict(q=FAKE, sq=1.0, sk=1.0, sv=1.0, ws=ctypes.c_void_p(0x100000), wsb=need, d=d,
                 scale=0.1, dq=FAKE)
        a.update(kw)
        return lib.fa_bwd_fp8(a["q"], FAKE, FAKE, a["sq"], a["sk"], a["sv"], FAKE, FAKE, FAKE,
                              a["dq"], FAKE, FAKE, a["ws"], a["wsb"], B, H, N, a["d"],
                              a["scale"], 1, None)

    assert f8b(q=None) == -1
    assert f8b(dq=None) == -1
    assert f8b(ws=None) == -1
    assert f8b(d=96) == -4
    assert f8b(sq=0.0) == -7
    assert f8b(sv=float("inf")) == -7
    assert f8b(sv=1e-39) == -7          # 1 / v_descale overflows
    assert f8b(scale=-1.0) == -7
    assert f8b(dq=ctypes.c_void_p(0x1004)) == -7
    assert f8b(wsb=need - 1) == -5
    assert f8b(ws=ctypes.c_void_p(0x100080)) == -5


def test_fwd_waves_validation(lib):
    def fw(**kw):
        a = dict(dtype=fa.FA_BF16, q=FAKE, d=128, waves=4, scale=0.1)
        a.update(kw)
        return lib.fa_fwd_waves(a["dtype"], a["q"], FAKE, FAKE, FAKE, FAKE, 1, 2, 64, a["d"],
                                a["scale"], 1, a["waves"], None)
    assert fw(q=None) == -1
    assert fw(dtype=fa.FA_F32) == -3
    assert fw(d=96) == -4
    assert fw(waves=2) == -7
    assert fw(waves=16) == -7
    assert fw(waves=-1) == -7
    assert fw(d=256, waves=8) == -7        # d = 256 runs four waves only
    assert fw(scale=0.0) == -7
    assert fw(q=ctypes.c_void_p(0x1008)) == -7


def test_probe_validation(lib):
    assert lib.fa_probe_mfma(None, 4, 10, None) == -1
    assert lib.fa_probe_mfma(FAKE, 0, 10, None) == -7
    assert lib.fa_probe_mfma(FAKE, 4, 0, None) == -7
    assert lib.fa_probe_mfma(FAKE, 65537, 10, None) == -7
    assert lib.fa_probe_mfma(ctypes.c_void_p(0x1004), 4, 10, None) == -7


def test_grid_bounds_rejected(lib):
    """Shapes whose one-dimensional launch grid would reach 2^32 work-items
    are refused with FA_ERR_SHAPE (HIP would refuse the launch instead)."""
    # B*H*ceil(N/32) must stay below 2^23: 2^23 heads of one token each
    assert fwd(lib, B=1 << 12, H=1 << 11, N=1, d=64) == -2
    assert fwd(lib, B=1 << 12, H=1 << 11, N=1, d=64, dtype=fa.FA_F32) == -2
    assert fwd(lib, B=1 << 11, H=1 << 11, N=33, d=64) == -2   # 2^22 heads x 2 blocks
    assert fa.fa_bwd_workspace_bytes(1 << 12, 1 << 11, 1, 64) == 0
    assert fa.fa_bwd_fp8_workspace_bytes(1 << 12, 1 << 11, 1, 64) == 0
    assert fa.fa_fwd_v1_workspace_bytes(1 << 12, 1 << 11, 1, 64) == 0
    # split-KV: 512 heads x 1024 query blocks x 256 key ranges x 256 work-items
    B, H, Nq, Nk, d = 1, 512, 32768, 32768, 64
    need = fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 256)
    assert need > 0
    assert lib.fa_fwd_splitkv(fa.FA_BF16, FAKE, FAKE, FAKE, FAKE, None, B, H, Nq, Nk, d, 0.1, 0,
                              256, ctypes.c_void_p(0x10000), need, None) == -2
    assert fa.fa_fwd_splitkv_workspace_bytes(1 << 12, 1 << 11, 1, 64, 64, 1) == 0
    # merge: rows * d / 4 work-items
    assert lib.fa_lse_merge(fa.FA_F32, 2, ctypes.c_void_p(0x10000), FAKE, FAKE, None, 1 << 30,
                            64, None) == -2
    # standard baseline: ceil(N/128)^2 score tiles of 256 work-items
    N = 1 << 19
    assert lib.fa_std_fwd(fa.FA_BF16, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10000),
                          fa.fa_std_workspace_bytes(1, 1, N, 64), 1, 1, N, 64, 0.1, 0,
                          None) == -2


def test_bwd_noalloc_validation(lib):
    """fa_bwd_noalloc validates like fa_bwd and refuses problems beyond its
    fixed scratch before any HIP call."""
    assert fa.fa_bwd_noalloc_max_rows() == 1 << 21

    def nb(**kw):
        a = dict(dtype=fa.FA_BF16, q=FAKE, dq=FAKE, B=1, H=2, N=64, d=64, scale=0.1)
        a.update(kw)
        return lib.fa_bwd_noalloc(a["dtype"], a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, a["dq"], FAKE,
                                  FAKE, a["B"], a["H"], a["N"], a["d"], a["scale"], 1, None)

    assert nb(q=None) == -1
    assert nb(dq=None) == -1
    assert nb(dtype=fa.FA_F32) == -3
    assert nb(d=96) == -4
    assert nb(B=0) == -2
    assert nb(scale=0.0) == -7
    assert nb(dq=ctypes.c_void_p(0x1008)) == -7
    assert nb(B=32, H=64, N=1025) == -8           # one row more than 2^21 (= 32*64*1024)
    assert nb(B=1, H=1, N=(1 << 21) + 1) == -8
    assert fa.fa_status_string(-8) != "unknown status"


def test_probe_dq_atomics_validation(lib):
    need = 1 * 2 * 256 * 128 * 4
    ws = ctypes.c_void_p(0x10000)

    def pr(**kw):
        a = dict(ws=ws, wsb=need, N=256, kb=128, mode=0)
        a.update(kw)
        return lib.fa_probe_dq_atomics(a["ws"], a["wsb"], 1, 2, a["N"], a["kb"], a["mode"], 1,
                                       None)

    assert pr(ws=None) == -1
    assert pr(N=100) == -2          # not a multiple of 64
    assert pr(N=320) == -2          # not a multiple of the key block
    assert pr(kb=64) == -7
    assert pr(mode=2) == -7
    assert pr(wsb=need - 4) == -5
    assert pr(ws=ctypes.c_void_p(0x10010)) == -5
