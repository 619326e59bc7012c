"""Exact scaled-dot-product attention on AMD MI355X (gfx950), FlashAttention-style.

The computation lives in ``libfa.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/fa.h``). This module is a thin ctypes binding with
the same entry-point names: it checks that torch tensors match the shapes the
C ABI will assume, passes their device pointers and the current HIP stream,
and raises ``FAError`` on a non-zero status. Every step of the attention runs
in the library's kernels; there is no fallback path. If the library has not
been built, calls raise ``RuntimeError``.

Entry points: ``fa_fwd``, ``fa_fwd_waves``, ``fa_fwd_fp8``, ``fa_bwd``,
``fa_bwd_stage``, ``fa_bwd_workspace_bytes``, ``fa_bwd_noalloc``,
``fa_bwd_noalloc_max_rows``, ``fa_bwd_fp8``,
``fa_bwd_fp8_workspace_bytes``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_workspace_bytes``, ``fa_lse_merge``, ``fa_fwd_v1``,
``fa_fwd_v1_workspace_bytes``, ``fa_std_fwd``, ``fa_std_workspace_bytes``,
``fa_probe_mfma``, ``fa_probe_dq_atomics``, ``fa_status_string``,
``fa_version``, ``fa_build_flags``; ``forward`` / ``backward`` /
``forward_fp8`` / ``backward_fp8`` / ``forward_splitkv`` / ``forward_v1`` /
``forward_standard`` allocate outputs with torch and call them.
``library_override(SERIAL_LIB_PATH)`` routes the wrappers through the
race-guard build for the duration of a ``with`` block.
"""

import contextlib
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SERIAL_LIB_PATH = os.path.join(PKG_DIR, "libfa_serial.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK = 0
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_DTYPE",
    -4: "FA_ERR_HEADDIM", -5: "FA_ERR_WORKSPACE", -6: "FA_ERR_HIP", -7: "FA_ERR_ARG",
    -8: "FA_ERR_TOO_LARGE",
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({fa_status_string(status)})")


def load_library(path=None):
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libfa.so not found at {path}; build it with "
                           "`python -m exact_io_aware_54_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_stage.argtypes = [i] + lib.fa_bwd.argtypes
    lib.fa_bwd_stage.restype = i
    lib.fa_bwd_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_rows.argtypes = []
    lib.fa_bwd_noalloc_max_rows.restype = sz
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_fwd_splitkv.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_lse_merge.argtypes = [i, i, vp, vp, vp, vp, i, i, vp]
    lib.fa_lse_merge.restype = i
    lib.fa_fwd_waves.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_waves.restype = i
    lib.fa_probe_mfma.argtypes = [vp, i, i, vp]
    lib.fa_probe_mfma.restype = i
    lib.fa_probe_dq_atomics.argtypes = [vp, sz, i, i, i, i, i, i, vp]
    lib.fa_probe_dq_atomics.restype = i
    lib.fa_bwd_fp8_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_fp8_workspace_bytes.restype = sz
    lib.fa_bwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f,
                               i, vp]
    lib.fa_bwd_fp8.restype = i
    lib.fa_fwd_v1_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_fwd_v1_workspace_bytes.restype = sz
    lib.fa_fwd_v1.argtypes = [i, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_fwd_v1.restype = i
    lib.fa_std_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_std_workspace_bytes.restype = sz
    lib.fa_std_fwd.argtypes = [i, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_std_fwd.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    lib.fa_build_flags.argtypes = []
    lib.fa_build_flags.restype = i
    _lib = lib
    return lib


@contextlib.contextmanager
def library_override(path):
    """Route every wrapper through another build of the library (such as the
    race-guard build libfa_serial.so) inside the block, then restore."""
    global _lib
    saved = _lib
    _lib = None
    try:
        yield load_library(path)
    finally:
        _lib = saved


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def fa_version():
    return load_library().fa_version()


def fa_build_flags():
    return load_library().fa_build_flags()


# ------------------------------------------------------------------ marshalling

def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_bhnd(name, t, shape, dtype=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")


def _raise(fn, st):
    if st != FA_OK:
        raise FAError(fn, st)


def fa_fwd(q, k, v, o, lse, scale, causal, stream=None):
    """Enqueue O = softmax(scale q k^T [causal]) v and LSE into ``o`` / ``lse``."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = lib.fa_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                    B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    _raise("fa_fwd", st)


def fa_fwd_waves(q, k, v, o, lse, scale, causal, waves, stream=None):
    """fa_fwd with the workgroup shape forced: waves 0 (built-in), 4 or 8."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = lib.fa_fwd_waves(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                          B, H, N, d, float(scale), int(bool(causal)), int(waves),
                          _stream(stream))
    _raise("fa_fwd_waves", st)


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, scale, causal, stream=None):
    """FP8 forward: q8/k8/v8 are uint8 E4M3 codes; o is bfloat16."""
    import torch
    lib = load_library()
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_bhnd(name, t, (B, H, N, d), torch.uint8)
    _check_bhnd("o", o, (B, H, N, d), torch.bfloat16)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), float(q_descale), float(k_descale),
                        float(v_descale), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                        int(bool(causal)), _stream(stream))
    _raise("fa_fwd_fp8", st)


def fa_bwd_workspace_bytes(B, H, N, d):
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, scale, causal, stream=None):
    """Enqueue dQ, dK, dV of <O, dO>; ``workspace`` is a uint8 device tensor."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_bwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                    B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    _raise("fa_bwd", st)


def fa_bwd_stage(stage, q, k, v, o, lse, do, dq, dk, dv, workspace, scale, causal, stream=None):
    """Enqueue one of fa_bwd's three launches (1 preprocess, 2 dK/dV, 3 dQ)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_bwd_stage(int(stage), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                          _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel(), B, H, N, d, float(scale), int(bool(causal)),
                          _stream(stream))
    _raise("fa_bwd_stage", st)


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal, stream=None):
    """fa_bwd without a workspace: the row terms live in the library's own
    per-device scratch (for callers that cannot allocate). Calls that overlap
    in time on one device race on that scratch."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = lib.fa_bwd_noalloc(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                            _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                            int(bool(causal)), _stream(stream))
    _raise("fa_bwd_noalloc", st)


def fa_bwd_noalloc_max_rows():
    return int(load_library().fa_bwd_noalloc_max_rows())


def fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits=0):
    return int(load_library().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, workspace, scale, causal, num_splits=0, stream=None):
    """Split-KV forward: q, o [B,H,Nq,d]; k, v [B,H,Nk,d]; lse [B,H,Nq] or None."""
    import torch
    lib = load_library()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_bhnd("q", q, (B, H, Nq, d), q.dtype)
    _check_bhnd("o", o, (B, H, Nq, d), q.dtype)
    _check_bhnd("k", k, (B, H, Nk, d), q.dtype)
    _check_bhnd("v", v, (B, H, Nk, d), q.dtype)
    if lse is not None:
        _check_bhnd("lse", lse, (B, H, Nq), torch.float32)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_fwd_splitkv(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                            None if lse is None else _ptr(lse), B, H, Nq, Nk, d, float(scale),
                            int(bool(causal)), int(num_splits), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    _raise("fa_fwd_splitkv", st)


def fa_lse_merge(o_parts, lse_parts, o, lse=None, stream=None):
    """Merge float32 parts o_parts [P, ..., d], lse_parts [P, ...] into o [..., d] (and lse)."""
    import torch
    lib = load_library()
    P, d = o_parts.shape[0], o_parts.shape[-1]
    rows = o_parts[0].numel() // d
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("o_parts and lse_parts must be float32")
    if tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError("lse_parts must have the shape of o_parts without its last dim")
    if tuple(o.shape) != tuple(o_parts.shape[1:]):
        raise ValueError("o must have the shape of one part")
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts), ("o", o)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() != rows or not lse.is_cuda):
        raise ValueError("lse must be a float32 device tensor with one value per row")
    st = lib.fa_lse_merge(_dtype_code(o), P, _ptr(o_parts), _ptr(lse_parts), _ptr(o),
                          None if lse is None else _ptr(lse), rows, d, _stream(stream))
    _raise("fa_lse_merge", st)


def fa_bwd_fp8_workspace_bytes(B, H, N, d):
    return int(load_library().fa_bwd_fp8_workspace_bytes(B, H, N, d))


def fa_bwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, do, dq, dk, dv, workspace,
               scale, causal, stream=None):
    """Gradients w.r.t. the dequantised fp8 inputs; o, do, dq, dk, dv are bfloat16."""
    import torch
    lib = load_library()
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_bhnd(name, t, (B, H, N, d), torch.uint8)
    for name, t in (("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, (B, H, N, d), torch.bfloat16)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_bwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), float(q_descale), float(k_descale),
                        float(v_descale), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                        _ptr(dv), _ptr(workspace), workspace.numel(), B, H, N, d, float(scale),
                        int(bool(causal)), _stream(stream))
    _raise("fa_bwd_fp8", st)


def fa_probe_mfma(sink, blocks, iters, stream=None):
    """Launch the MFMA-rate / clock probe; sink is an int64 device tensor of 3*blocks."""
    import torch
    if sink.dtype != torch.int64 or not sink.is_cuda or sink.numel() < 3 * blocks:
        raise ValueError("sink must be an int64 device tensor of at least 3*blocks elements")
    _raise("fa_probe_mfma", load_library().fa_probe_mfma(_ptr(sink), int(blocks), int(iters),
                                                          _stream(stream)))


def fa_probe_dq_atomics(ws, B, H, N, key_block, mode, causal, stream=None):
    """Launch the dQ-atomics probe (mode 0 atomics, 1 plain stores); ws is float32 [B*H*N*128]."""
    import torch
    if ws.dtype != torch.float32 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous float32 device tensor")
    _raise("fa_probe_dq_atomics", load_library().fa_probe_dq_atomics(
        _ptr(ws), ws.numel() * 4, B, H, N, int(key_block), int(mode), int(bool(causal)),
        _stream(stream)))


def fa_fwd_v1_workspace_bytes(B, H, N, d):
    return int(load_library().fa_fwd_v1_workspace_bytes(B, H, N, d))


def fa_fwd_v1(q, k, v, o, lse, workspace, scale, causal, stream=None):
    """First-generation loop order (K/V blocks outer, O/m/l through memory)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    if lse is not None:
        _check_bhnd("lse", lse, (B, H, N), torch.float32)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_fwd_v1(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                       None if lse is None else _ptr(lse), _ptr(workspace), workspace.numel(),
                       B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    _raise("fa_fwd_v1", st)


def fa_std_workspace_bytes(B, H, N, d):
    return int(load_library().fa_std_workspace_bytes(B, H, N, d))


def fa_std_fwd(q, k, v, o, workspace, scale, causal, stream=None):
    """Standard attention (S and P materialised in ``workspace``) into ``o``."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, (B, H, N, d), q.dtype)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be a uint8 device tensor")
    st = lib.fa_std_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(workspace),
                        workspace.numel(), B, H, N, d, float(scale), int(bool(causal)),
                        _stream(stream))
    _raise("fa_std_fwd", st)


# ------------------------------------------------- allocate-and-call conveniences

def forward(q, k, v, scale=None, causal=False):
    """Allocate O and LSE with torch and run fa_fwd. Returns (o, lse)."""
    import torch
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], device=q.device, dtype=torch.float32)
    fa_fwd(q, k, v, o, lse, scale, causal)
    return o, lse


def forward_splitkv(q, k, v, scale=None, causal=False, num_splits=0):
    """Allocate O, LSE and the workspace with torch and run fa_fwd_splitkv."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = d ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    ws = torch.empty(max(1, fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits)),
                     device=q.device, dtype=torch.uint8)
    fa_fwd_splitkv(q, k, v, o, lse, ws, scale, causal, num_splits)
    return o, lse


def backward_fp8(q8, k8, v8, descales, o, lse, do, scale=None, causal=False):
    """Allocate dQ, dK, dV (bfloat16) and the workspace with torch and run fa_bwd_fp8."""
    import torch
    B, H, N, d = q8.shape
    scale = d ** -0.5 if scale is None else scale
    dq, dk, dv = (torch.empty((B, H, N, d), device=q8.device, dtype=torch.bfloat16)
                  for _ in range(3))
    ws = torch.empty(fa_bwd_fp8_workspace_bytes(B, H, N, d), device=q8.device, dtype=torch.uint8)
    fa_bwd_fp8(q8, k8, v8, descales[0], descales[1], descales[2], o, lse, do, dq, dk, dv, ws,
               scale, causal)
    return dq, dk, dv


def forward_v1(q, k, v, scale=None, causal=False):
    """Allocate O, LSE and the workspace with torch and run fa_fwd_v1."""
    import torch
    B, H, N, d = q.shape
    scale = d ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    ws = torch.empty(fa_fwd_v1_workspace_bytes(B, H, N, d), device=q.device, dtype=torch.uint8)
    fa_fwd_v1(q, k, v, o, lse, ws, scale, causal)
    return o, lse


def forward_standard(q, k, v, scale=None, causal=False):
    """Allocate O and the N x N workspace with torch and run fa_std_fwd."""
    import torch
    B, H, N, d = q.shape
    scale = d ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    ws = torch.empty(fa_std_workspace_bytes(B, H, N, d), device=q.device, dtype=torch.uint8)
    fa_std_fwd(q, k, v, o, ws, scale, causal)
    return o


def forward_fp8(q8, k8, v8, descales, scale=None, causal=False):
    import torch
    scale = q8.shape[-1] ** -0.5 if scale is None else scale
    o = torch.empty(q8.shape, device=q8.device, dtype=torch.bfloat16)
    lse = torch.empty(q8.shape[:-1], device=q8.device, dtype=torch.float32)
    fa_fwd_fp8(q8, k8, v8, descales[0], descales[1], descales[2], o, lse, scale, causal)
    return o, lse


def workspace_for(q):
    import torch
    B, H, N, d = q.shape
    return torch.empty(fa_bwd_workspace_bytes(B, H, N, d), device=q.device, dtype=torch.uint8)


def backward(q, k, v, o, lse, do, scale=None, causal=False, workspace=None):
    """Allocate dQ, dK, dV (and a workspace if none is given) and run fa_bwd."""
    import torch
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = workspace_for(q) if workspace is None else workspace
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal)
    return dq, dk, dv
