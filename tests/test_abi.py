"""C-ABI checks that need no GPU: the libraries load, export every entry point
declared in include/fa_mi355x.h and include/fa_micro.h, and reject bad
arguments before any HIP call.

Every call made here fails validation, so no kernel is launched. The calls
pass fake device addresses, so they run only on a host without a GPU (no
/dev/kfd): there, even a validation check that regressed could not launch a
kernel on those addresses; on a GPU host they are skipped.
"""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_13_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

# Fake device addresses: non-null and 16-byte aligned (never dereferenced).
P = 0x100000
MIS = 0x100008  # 8-byte aligned only

no_gpu_only = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                 reason="fake device addresses are passed only where no GPU exists")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_poison_build_exports_every_declared_symbol():
    L = ctypes.CDLL(fa.LIB_POISON_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_micro_library_exports_every_declared_symbol():
    from exact_tiled_attention_13_amd import micro
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa_micro.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+([a-z_0-9]+)\s*\(", text, flags=re.M)))
    assert names == ["fa_micro_atomic_add", "fa_micro_exp2", "fa_micro_fp8_dot", "fa_micro_mfma_bf16",
                     "fa_micro_mfma_valu"]
    L = ctypes.CDLL(micro.LIB_MICRO)
    for name in names:
        assert hasattr(L, name), name


@no_gpu_only
def test_noalloc_rejects_bad_arguments_before_any_hip_call():
    L = fa.lib()
    args = lambda **kw: [kw.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")] + \
        [kw.get("B", 1), kw.get("H", 2), kw.get("N", 100), kw.get("d", 64), 0, 0.125, None]
    assert L.attn_bwd_noalloc(*args(q=0)) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_noalloc(*args(dv=MIS)) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_noalloc(*args(d=96)) == fa.FA_ERR_UNSUPPORTED
    assert L.attn_bwd_noalloc(*args(N=0)) == fa.FA_ERR_INVALID_ARG
    # 64 heads of 65536 tokens need 32 MiB of statistics: beyond the static scratch.
    assert fa.attn_bwd_workspace_size(1, 64, 65536, 64) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert L.attn_bwd_noalloc(*args(H=64, N=65536)) == fa.FA_ERR_WORKSPACE
    assert fa.attn_bwd_workspace_size(1, 16, 131072, 64) <= fa.FA_NOALLOC_SCRATCH_BYTES


@no_gpu_only
def test_micro_rejects_bad_arguments():
    from exact_tiled_attention_13_amd import micro
    L = micro.lib()
    assert L.fa_micro_mfma_bf16(0, P, 4, 2, 0, None) == 1
    assert L.fa_micro_mfma_bf16(P, P, 4, 3, 0, None) == 1       # odd iteration count
    assert L.fa_micro_mfma_bf16(P, P, 4, 2, 6, None) == 1       # unknown operand mode
    assert L.fa_micro_exp2(P, P, 0, 1, None) == 1
    assert L.fa_micro_mfma_valu(P, P, 4, 10, 3, 0, None) == 1   # unsupported mix
    assert L.fa_micro_fp8_dot(P, P, P, 1, 65, None) == 1
    assert L.fa_micro_fp8_dot(P, MIS, P, 1, 1, None) == 1
    assert L.fa_micro_atomic_add(P, 100, 1, None) == 1          # not a multiple of 256


def test_status_strings():
    assert fa.status_string(0) == "FA_OK"
    assert fa.status_string(1) == "FA_ERR_INVALID_ARG"
    assert fa.status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.status_string(3) == "FA_ERR_WORKSPACE"
    assert fa.status_string(4) == "FA_ERR_HIP"
    assert fa.status_string(99) == "FA_ERR_UNKNOWN"


def fwd(fn="attn_fwd", q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, causal=0, scale=0.125):
    return getattr(fa.lib(), fn)(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@no_gpu_only
@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_fp32"])
def test_forward_rejects_bad_arguments(fn):
    assert fwd(fn, q=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, lse=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, o=MIS) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, q=P, B=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, H=-1) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, N=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, scale=float("inf")) == fa.FA_ERR_INVALID_ARG
    assert fwd(fn, N=1 << 24, H=1024, d=128) == fa.FA_ERR_INVALID_ARG  # N*H*d >= 2^31
    for d in (0, 32, 96, 256):
        assert fwd(fn, d=d) == fa.FA_ERR_UNSUPPORTED
    # Size checks come before pointer checks: a bad size with a null pointer is still INVALID_ARG.
    assert fwd(fn, q=0, d=96) == fa.FA_ERR_UNSUPPORTED


def bwd(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, ws_bytes=1 << 20, B=1, H=1, N=16, d=64,
        causal=0, scale=0.125):
    return fa.lib().attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, N, d, causal, scale, None)


@no_gpu_only
def test_backward_rejects_bad_arguments():
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(**{name: 0}) == fa.FA_ERR_INVALID_ARG, name
        assert bwd(**{name: MIS}) == fa.FA_ERR_INVALID_ARG, name
    assert bwd(B=0) == fa.FA_ERR_INVALID_ARG
    assert bwd(scale=float("-inf")) == fa.FA_ERR_INVALID_ARG
    assert bwd(d=80) == fa.FA_ERR_UNSUPPORTED
    assert bwd(ws=0) == fa.FA_ERR_WORKSPACE
    assert bwd(ws=MIS) == fa.FA_ERR_WORKSPACE
    need = fa.attn_bwd_workspace_size(1, 1, 16, 64, False)
    assert bwd(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE


def test_workspace_size():
    # two fp32 arrays [B, H, 64 * ceil(N / 64)], rounded up to 256 bytes
    assert fa.attn_bwd_workspace_size(1, 1, 16, 64, False) == 512
    assert fa.attn_bwd_workspace_size(4, 16, 4096, 128, True) == 2 * 4 * 16 * 4096 * 4
    assert fa.attn_bwd_workspace_size(1, 1, 65, 64, False) == 1024
    assert fa.attn_bwd_workspace_size(3, 1, 1, 64, False) == 1536  # 2 * 3 * 64 * 4, already a multiple of 256
    assert fa.attn_bwd_workspace_size(0, 1, 16, 64, False) == 0
    assert fa.attn_bwd_workspace_size(1, 1, 16, 96, False) == 0


@no_gpu_only
def test_backward_stages_reject_bad_arguments():
    L = fa.lib()
    need = fa.attn_bwd_workspace_size(1, 1, 16, 64, False)
    # attn_bwd_prep(o, dO, lse, ws, ws_bytes, B, H, N, d, stream)
    assert L.attn_bwd_prep(0, P, P, P, need, 1, 1, 16, 64, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_prep(P, P, 0, P, need, 1, 1, 16, 64, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_prep(P, P, P, P, need - 1, 1, 1, 16, 64, None) == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_prep(P, P, P, 0, need, 1, 1, 16, 64, None) == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_prep(P, P, P, P, need, 1, 1, 16, 48, None) == fa.FA_ERR_UNSUPPORTED
    # attn_bwd_dkdv(q, k, v, dO, ws, ws_bytes, dk, dv, B, H, N, d, causal, scale, stream)
    assert L.attn_bwd_dkdv(P, P, P, P, P, need, 0, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dkdv(P, P, P, P, P, need - 1, P, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_dkdv(P, P, MIS, P, P, need, P, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dkdv(P, P, P, P, P, need, P, P, 1, 1, 16, 64, 0, float("nan"), None) == fa.FA_ERR_INVALID_ARG
    # attn_bwd_dq(q, k, v, dO, ws, ws_bytes, dq, B, H, N, d, causal, scale, stream)
    assert L.attn_bwd_dq(P, P, P, P, P, need, 0, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dq(P, P, P, P, 0, need, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_dq(P, P, P, P, P, need, P, 1, 0, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    # attn_bwd_dq_prep(q, k, v, o, dO, lse, ws, ws_bytes, dq, B, H, N, d, causal, scale, stream)
    assert L.attn_bwd_dq_prep(P, P, P, 0, P, P, P, need, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dq_prep(P, P, P, P, P, 0, P, need, P, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dq_prep(P, P, P, P, P, MIS, P, need, P, 1, 1, 16, 64, 0, 0.125, None) \
        == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dq_prep(P, P, P, P, P, P, P, need, 0, 1, 1, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_dq_prep(P, P, P, P, P, P, P, need - 1, P, 1, 1, 16, 64, 0, 0.125, None) \
        == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_dq_prep(P, P, P, P, P, P, P, need, P, 1, 1, 16, 48, 0, 0.125, None) == fa.FA_ERR_UNSUPPORTED


@no_gpu_only
def test_gqa_rejects_bad_head_counts():
    L = fa.lib()
    # attn_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream)
    assert L.attn_fwd_gqa(P, P, P, P, P, 1, 4, 3, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_fwd_gqa(P, P, P, P, P, 1, 4, 0, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_fwd_gqa(P, P, P, P, P, 1, 4, -2, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_fwd_gqa(P, P, P, P, P, 1, 4, 2, 16, 96, 0, 0.125, None) == fa.FA_ERR_UNSUPPORTED
    assert L.attn_fwd_gqa(P, P, 0, P, P, 1, 4, 2, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    need = fa.attn_bwd_workspace_size(1, 4, 16, 64, False)
    # attn_bwd_gqa(q, k, v, o, dO, lse, dq, dk, dv, ws, ws_bytes, B, H, Hkv, N, d, causal, scale, stream)
    args = [P] * 10 + [need]
    assert L.attn_bwd_gqa(*args, 1, 4, 3, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_gqa(*args, 1, 4, 0, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG
    assert L.attn_bwd_gqa(*([P] * 10), need - 1, 1, 4, 2, 16, 64, 0, 0.125, None) == fa.FA_ERR_WORKSPACE
    assert L.attn_bwd_gqa(*([P] * 6), 0, P, P, P, need, 1, 4, 2, 16, 64, 0, 0.125, None) == fa.FA_ERR_INVALID_ARG


def test_gqa_workspace_size():
    # Never below the unsplit workspace; equal to it when K/V heads = query heads
    # or the grid is already large; a multiple of the fp32 partial dK, dV more
    # when split; 0 for rejected arguments.
    for B, H, Hkv, N, d, c in [(1, 16, 2, 16384, 128, 1), (1, 16, 2, 16384, 128, 0), (2, 8, 1, 17, 64, 0),
                               (1, 8, 8, 4096, 128, 1), (16, 32, 8, 1024, 128, 1)]:
        base = fa.attn_bwd_workspace_size(B, H, N, d, c)
        full = fa.attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, c)
        assert full >= base > 0
        part = 2 * B * N * Hkv * d * 4
        extra = full - base
        assert extra == 0 or (extra % part == 0 and (H // Hkv) % (extra // part) == 0 and extra // part > 1)
        if Hkv == H:
            assert full == base
    # 16 query heads on 2 K/V heads at 16k tokens: one unsplit workgroup per CU
    # under the causal mask would leave the first key block alone setting the time.
    assert fa.attn_bwd_gqa_workspace_size(1, 16, 2, 16384, 128, 1) > fa.attn_bwd_workspace_size(1, 16, 16384, 128, 1)
    assert fa.attn_bwd_gqa_workspace_size(1, 16, 2, 16384, 128, 0) == fa.attn_bwd_workspace_size(1, 16, 16384, 128, 0)
    assert fa.attn_bwd_gqa_workspace_size(1, 4, 3, 16, 64, 0) == 0
    assert fa.attn_bwd_gqa_workspace_size(1, 4, 2, 16, 96, 0) == 0
    assert fa.attn_bwd_gqa_workspace_size(1, 4, 2, 0, 64, 0) == 0


def dec(q=P, k=P, v=P, o=P, lse=P, ws=P, wsb=1 << 30, B=1, H=8, Hkv=2, Nq=1, Nk=100, d=128, causal=0, scale=0.1):
    return fa.lib().attn_decode(q, k, v, o, lse, ws, wsb, B, H, Hkv, Nq, Nk, d, causal, scale, None)


def test_decode_workspace_size():
    L = fa.lib()
    n = L.attn_decode_workspace_size(2, 8, 2, 3, 1000, 128)
    assert n > 0 and n % 256 == 0
    # At least the per-chunk outputs and LSE of every query row of the workgroups that cover the cache.
    assert n >= 2 * 2 * (4 * 3) * (128 + 1) * 4
    assert L.attn_decode_workspace_size(1, 8, 3, 1, 10, 128) == 0      # H not a multiple of Hkv
    assert L.attn_decode_workspace_size(1, 64, 1, 1, 10, 128) == 0     # 64 query rows per K/V head
    assert L.attn_decode_workspace_size(1, 8, 2, 1, 10, 96) == 0       # head dim
    assert L.attn_decode_workspace_size(1, 8, 2, 0, 10, 128) == 0


@no_gpu_only
def test_decode_rejects_bad_arguments():
    assert dec(q=0) == fa.FA_ERR_INVALID_ARG
    assert dec(lse=MIS) == fa.FA_ERR_INVALID_ARG
    assert dec(B=0) == fa.FA_ERR_INVALID_ARG
    assert dec(Nq=0) == fa.FA_ERR_INVALID_ARG
    assert dec(Nk=0) == fa.FA_ERR_INVALID_ARG
    assert dec(Hkv=3) == fa.FA_ERR_INVALID_ARG
    assert dec(Hkv=0) == fa.FA_ERR_INVALID_ARG
    assert dec(scale=float("inf")) == fa.FA_ERR_INVALID_ARG
    assert dec(causal=1, Nq=8, Nk=4, H=2, Hkv=2) == fa.FA_ERR_INVALID_ARG   # more new tokens than cached keys
    assert dec(d=80) == fa.FA_ERR_UNSUPPORTED
    assert dec(H=32, Hkv=1, Nq=2) == fa.FA_ERR_UNSUPPORTED                 # 64 query rows per K/V head
    assert dec(ws=0) == fa.FA_ERR_WORKSPACE
    assert dec(ws=MIS) == fa.FA_ERR_WORKSPACE
    assert dec(wsb=16) == fa.FA_ERR_WORKSPACE


def f8(q=P, k=P, vt=P, ldv=128, dq=1.0, dk=1.0, dv=1.0, o=P, lse=P, B=1, H=2, N=100, d=128, causal=0, scale=0.1):
    return fa.lib().attn_fwd_fp8(q, k, vt, ldv, dq, dk, dv, o, lse, B, H, N, d, causal, scale, None)


@no_gpu_only
def test_fp8_rejects_bad_arguments():
    assert f8(q=0) == fa.FA_ERR_INVALID_ARG
    assert f8(vt=MIS) == fa.FA_ERR_INVALID_ARG
    assert f8(N=0) == fa.FA_ERR_INVALID_ARG
    assert f8(dq=0.0) == fa.FA_ERR_INVALID_ARG
    assert f8(dk=-1.0) == fa.FA_ERR_INVALID_ARG
    assert f8(dv=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert f8(ldv=100) == fa.FA_ERR_INVALID_ARG        # fewer than 64 * ceil(N / 64) bytes per row
    assert f8(ldv=136, N=100) == fa.FA_ERR_INVALID_ARG  # ldv = 136 covers N but is not a multiple of 16... (136 % 16 = 8)
    assert f8(scale=float("inf")) == fa.FA_ERR_INVALID_ARG
    assert f8(d=64) == fa.FA_ERR_UNSUPPORTED
