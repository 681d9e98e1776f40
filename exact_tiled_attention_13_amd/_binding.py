"""ctypes binding of libfa_mi355x.so (C ABI in include/fa_mi355x.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the attention computation runs in the library's HIP
kernels. There is no fallback: if the library is missing or a call is
rejected, an exception is raised.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The attention library. FA_MI355X_LIB may name another build of the same
# sources instead (for instance libfa_mi355x_ldspoison.so, the race-check
# build whose kernels fill their LDS with NaN before use).
LIB_PATH = os.environ.get("FA_MI355X_LIB") or os.path.join(_PKG, "libfa_mi355x.so")
LIB_POISON_PATH = os.path.join(_PKG, "libfa_mi355x_ldspoison.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4

EXPORTED = ("attn_fwd", "attn_fwd_fp32", "attn_bwd", "attn_bwd_workspace_size", "attn_bwd_prep",
            "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_prep", "attn_fwd_gqa", "attn_bwd_gqa", "attn_bwd_gqa_workspace_size",
            "attn_decode_workspace_size",
            "attn_decode", "attn_fwd_fp8", "attn_bwd_noalloc", "fa_status_string")

FA_NOALLOC_SCRATCH_BYTES = 16 << 20     # include/fa_mi355x.h

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    """A libfa_mi355x entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the shared library once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = _load(LIB_PATH)
        return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Route every call of this module to the library at `path` (another build of the same sources, e.g.
    LIB_POISON_PATH) until the block exits."""
    global _lib
    alt = _load(path)
    with _lock:
        prev = _lib
        _lib = alt
    try:
        yield alt
    finally:
        with _lock:
            _lib = prev


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_tiled_attention_13_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(path)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_fwd.restype = ci
    L.attn_fwd_fp32.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_fwd_fp32.restype = ci
    L.attn_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_bwd.argtypes = [vp] * 9 + [vp, sz] + [ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd.restype = ci
    L.attn_bwd_prep.argtypes = [vp, vp, vp, vp, sz, ci, ci, ci, ci, vp]
    L.attn_bwd_prep.restype = ci
    L.attn_bwd_dkdv.argtypes = [vp] * 5 + [sz, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd_dkdv.restype = ci
    L.attn_bwd_dq.argtypes = [vp] * 5 + [sz, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd_dq.restype = ci
    L.attn_bwd_dq_prep.argtypes = [vp] * 7 + [sz, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd_dq_prep.restype = ci
    L.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    L.attn_fwd_gqa.restype = ci
    L.attn_bwd_gqa.argtypes = [vp] * 9 + [vp, sz] + [ci, ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd_gqa.restype = ci
    L.attn_bwd_gqa_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_bwd_gqa_workspace_size.restype = sz
    L.attn_decode_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_decode_workspace_size.restype = sz
    L.attn_decode.argtypes = [vp] * 5 + [vp, sz] + [ci, ci, ci, ci, ci, ci, ci, cf, vp]
    L.attn_decode.restype = ci
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, ci, cf, cf, cf, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    L.attn_fwd_fp8.restype = ci
    L.attn_bwd_noalloc.argtypes = [vp] * 9 + [ci, ci, ci, ci, ci, cf, vp]
    L.attn_bwd_noalloc.restype = ci
    L.fa_status_string.argtypes = [ci]
    L.fa_status_string.restype = ctypes.c_char_p
    return L


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn: str, status: int):
    if status != FA_OK:
        raise FaError(fn, status)


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected [B, N, H, d] tensors, got shape {tuple(q.shape)}")
    B, N, H, d = q.shape
    return B, N, H, d


def _expect(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None):
    """bf16 forward. q, k, v: contiguous bf16 [B, N, H, d] on one GPU. Returns (o, lse)."""
    B, N, H, d = _shape(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _expect("o", o, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    s = default_scale(d) if scale is None else float(scale)
    st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), s,
                        _stream(dev))
    _check("attn_fwd", st)
    return o, lse


def attn_fwd_fp32(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None):
    """fp32 forward. q, k, v: contiguous fp32 [B, N, H, d]. Returns (o, lse)."""
    B, N, H, d = _shape(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(name, t, (B, N, H, d), torch.float32, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _expect("o", o, (B, N, H, d), torch.float32, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    s = default_scale(d) if scale is None else float(scale)
    st = lib().attn_fwd_fp32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), s,
                             _stream(dev))
    _check("attn_fwd_fp32", st)
    return o, lse


def attn_bwd_workspace_size(B: int, H: int, N: int, d: int, causal: bool = False) -> int:
    return int(lib().attn_bwd_workspace_size(B, H, N, d, int(bool(causal))))


def attn_bwd(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward. Returns (dq, dk, dv), each contiguous bf16 [B, N, H, d]."""
    B, N, H, d = _shape(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    need = attn_bwd_workspace_size(B, H, N, d, causal)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    s = default_scale(d) if scale is None else float(scale)
    st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, N, d,
                        int(bool(causal)), s, _stream(dev))
    _check("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
                     dq=None, dk=None, dv=None):
    """attn_bwd with the workspace in the library's static device scratch (no workspace argument; the C
    call allocates nothing). Outputs are allocated here unless given. Returns (dq, dk, dv)."""
    B, N, H, d = _shape(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    s = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(dev):
        st = lib().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, N, d, int(bool(causal)), s, _stream(dev))
    _check("attn_bwd_noalloc", st)
    return dq, dk, dv


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def workspace(B: int, H: int, N: int, d: int, device) -> torch.Tensor:
    """A workspace tensor of attn_bwd_workspace_size bytes (uint8) on `device`."""
    return torch.empty(attn_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=device)


def attn_bwd_gqa_workspace_size(B: int, H: int, Hkv: int, N: int, d: int, causal: bool = False) -> int:
    """Bytes of workspace that let attn_bwd_gqa split the query heads of a K/V head (0 if rejected)."""
    return int(lib().attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, int(bool(causal))))


def workspace_gqa(B: int, H: int, Hkv: int, N: int, d: int, causal: bool, device) -> torch.Tensor:
    """A workspace tensor of attn_bwd_gqa_workspace_size bytes (uint8) on `device`."""
    return torch.empty(max(attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, causal), 256), dtype=torch.uint8,
                       device=device)


def attn_bwd_prep(o, do, lse, ws=None):
    """Fill the backward workspace (D_i and LSE_i * log2 e). Returns the workspace."""
    B, N, H, d = _shape(o)
    dev = o.device
    _expect("o", o, (B, N, H, d), torch.bfloat16, dev)
    _expect("do", do, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    ws = workspace(B, H, N, d, dev) if ws is None else ws
    _check("attn_bwd_prep", lib().attn_bwd_prep(_ptr(o), _ptr(do), _ptr(lse), _ptr(ws), _nbytes(ws),
                                                B, H, N, d, _stream(dev)))
    return ws


def attn_bwd_dkdv(q, k, v, do, ws, causal: bool = False, scale: float | None = None, dk=None, dv=None):
    """dK and dV from the forward inputs, dO and a workspace filled by attn_bwd_prep. Returns (dk, dv)."""
    B, N, H, d = _shape(q)
    dev = q.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dk", dk), ("dv", dv)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_bwd_dkdv", lib().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(ws), _nbytes(ws),
                                                _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), s,
                                                _stream(dev)))
    return dk, dv


def attn_bwd_dq(q, k, v, do, ws, causal: bool = False, scale: float | None = None, dq=None):
    """dQ from the forward inputs, dO and a workspace filled by attn_bwd_prep. Returns dq."""
    B, N, H, d = _shape(q)
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dq", dq)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_bwd_dq", lib().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(ws), _nbytes(ws), _ptr(dq),
                                            B, H, N, d, int(bool(causal)), s, _stream(dev)))
    return dq


def attn_bwd_dq_prep(q, k, v, o, do, lse, ws=None, causal: bool = False, scale: float | None = None, dq=None):
    """dQ, and the workspace's row statistics for attn_bwd_dkdv, in one launch (attn_bwd_prep's work fused
    into attn_bwd_dq). Returns (dq, ws)."""
    B, N, H, d = _shape(q)
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    ws = workspace(B, H, N, d, dev) if ws is None else ws
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_bwd_dq_prep", lib().attn_bwd_dq_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                                      _ptr(ws), _nbytes(ws), _ptr(dq), B, H, N, d,
                                                      int(bool(causal)), s, _stream(dev)))
    return dq, ws


def _kv_heads(q, k):
    B, N, H, d = _shape(q)
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"k: expected [B, N, Hkv, d] = [{B}, {N}, Hkv, {d}], got {tuple(k.shape)}")
    return B, N, H, int(k.shape[2]), d


def attn_fwd_gqa(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None):
    """Grouped-query forward: q [B, N, H, d], k, v [B, N, Hkv, d] bf16 (H a multiple of Hkv). Returns (o, lse)."""
    B, N, H, Hkv, d = _kv_heads(q, k)
    dev = q.device
    _expect("q", q, (B, N, H, d), torch.bfloat16, dev)
    for name, t in (("k", k), ("v", v)):
        _expect(name, t, (B, N, Hkv, d), torch.bfloat16, dev)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _expect("o", o, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_fwd_gqa", lib().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                              int(bool(causal)), s, _stream(dev)))
    return o, lse


def attn_bwd_gqa(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
                 dq=None, dk=None, dv=None, workspace=None):
    """Grouped-query backward. Returns (dq [B, N, H, d], dk, dv [B, N, Hkv, d]), bf16."""
    B, N, H, Hkv, d = _kv_heads(q, k)
    dev = q.device
    for name, t in (("q", q), ("o", o), ("do", do)):
        _expect(name, t, (B, N, H, d), torch.bfloat16, dev)
    for name, t in (("k", k), ("v", v)):
        _expect(name, t, (B, N, Hkv, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _expect("dq", dq, (B, N, H, d), torch.bfloat16, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        _expect(name, t, (B, N, Hkv, d), torch.bfloat16, dev)
    if workspace is None:
        workspace = workspace_gqa(B, H, Hkv, N, d, causal, dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_bwd_gqa", lib().attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                              _ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace), B, H, Hkv,
                                              N, d, int(bool(causal)), s, _stream(dev)))
    return dq, dk, dv


def attn_decode_workspace_size(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    """Bytes of scratch attn_decode needs for this shape (0 if the library rejects the shape)."""
    return int(lib().attn_decode_workspace_size(B, H, Hkv, Nq, Nk, d))


def attn_decode(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None, ws=None):
    """Decoding against a cache: q [B, Nq, H, d], k, v [B, Nk, Hkv, d] bf16. Returns (o, lse).

    Query i is the token at position Nk - Nq + i (causal: it sees keys <= that
    position). ``ws`` is an optional uint8 workspace of at least
    attn_decode_workspace_size(...) bytes; one is allocated when omitted.
    """
    B, Nq, H, d = _shape(q)
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k: expected [B, Nk, Hkv, d] = [{B}, Nk, Hkv, {d}], got {tuple(k.shape)}")
    Nk, Hkv = int(k.shape[1]), int(k.shape[2])
    dev = q.device
    _expect("q", q, (B, Nq, H, d), torch.bfloat16, dev)
    for name, t in (("k", k), ("v", v)):
        _expect(name, t, (B, Nk, Hkv, d), torch.bfloat16, dev)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev) if lse is None else lse
    _expect("o", o, (B, Nq, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, Nq), torch.float32, dev)
    if ws is None:
        ws = torch.empty(max(attn_decode_workspace_size(B, H, Hkv, Nq, Nk, d), 256), dtype=torch.uint8, device=dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_decode", lib().attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), _nbytes(ws),
                                            B, H, Hkv, Nq, Nk, d, int(bool(causal)), s, _stream(dev)))
    return o, lse


def _bytes8(name, t, shape, device):
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(t.shape) != tuple(shape) \
            or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous float8_e4m3fn (or uint8) {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def attn_fwd_fp8(q8, k8, vt8, q_descale: float, k_descale: float, v_descale: float, causal: bool = False,
                 scale: float | None = None, o=None, lse=None):
    """FP8 (E4M3) forward. q8, k8 [B, N, H, d]; vt8 = V transposed per head [B, H, d, ldv] (keys
    contiguous, zero padding past N, ldv a multiple of 64 covering N). Returns (o bf16, lse fp32)."""
    B, N, H, d = _shape(q8)
    dev = q8.device
    _bytes8("q8", q8, (B, N, H, d), dev)
    _bytes8("k8", k8, (B, N, H, d), dev)
    if vt8.dim() != 4:
        raise ValueError(f"vt8: expected [B, H, d, ldv], got {tuple(vt8.shape)}")
    ldv = int(vt8.shape[3])
    _bytes8("vt8", vt8, (B, H, d, ldv), dev)
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _expect("o", o, (B, N, H, d), torch.bfloat16, dev)
    _expect("lse", lse, (B, H, N), torch.float32, dev)
    s = default_scale(d) if scale is None else float(scale)
    _check("attn_fwd_fp8", lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), ldv, float(q_descale),
                                              float(k_descale), float(v_descale), _ptr(o), _ptr(lse), B, H, N, d,
                                              int(bool(causal)), s, _stream(dev)))
    return o, lse
