"""Seeded synthetic inputs and the named attention workloads.

This module holds no attention arithmetic. It is the only code that both the
HIP path's callers (tests, bench) and the CPU oracle's callers share: it draws
the tensors, and each side then computes on identical values.

Recipe: a CPU ``torch.Generator`` seeded per workload draws Q, then K, then V,
then dO, each ``randn(B, N, H, d)`` in float32 (iid N(0, 1), no structure),
then rounds to bfloat16 with round-to-nearest-even unless the workload is
fp32. Layout is ``[B, N, H, d]``, d fastest, contiguous.

The workload sweep follows the kernel benchmark that the page
"FlashAttention-2: atención eficiente en GPU para contextos largos" describes
in section "Qué significa la mejora de aproximadamente dos veces": sequence
lengths from 512 to about 16k, head dimensions 64 and 128, with and without
the causal mask, at 16k tokens per batch. It names no dataset; these seeded
tensors stand in for its inputs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" or "bf16"
    B: int
    H: int
    N: int
    d: int
    causal: tuple       # masks the workload is run with
    backward: bool
    seed: int
    Hkv: int = 0        # K/V heads for grouped-query attention (0: same as H)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to fp32 (the value the library receives)."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def tokens(self) -> int:
        return self.B * self.N


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_fp32_b1_h2_n128_d64", "fp32", 1, 2, 128, 64, (False,), False, 1001),
        Workload("fwd_bf16_b32_h32_n512_d64", "bf16", 32, 32, 512, 64, (False, True), False, 1002),
        Workload("fwd_bf16_b8_h16_n2048_d128", "bf16", 8, 16, 2048, 128, (True,), False, 1003),
        Workload("fwd_bf16_b1_h16_n16384_d128", "bf16", 1, 16, 16384, 128, (False, True), False, 1004),
        Workload("bwd_bf16_b4_h16_n4096_d128", "bf16", 4, 16, 4096, 128, (True,), True, 1005),
    ]
}

# Backward timed at the long-context shape (batch 1, 16 heads, 16k tokens, d 128).
BWD_LONG = Workload("bwd_bf16_b1_h16_n16384_d128", "bf16", 1, 16, 16384, 128, (False, True), True, 1004)

# The head-dim-64 point of the same 16k-token sweep at its longest sequence
# (H * d = 2048 as in every other workload); reported beside the main step.
LONG_D64 = Workload("bwd_bf16_b1_h32_n16384_d64", "bf16", 1, 32, 16384, 64, (False, True), True, 1006)

# Grouped-query attention at the long-context shape: 16 query heads sharing
# 2 K/V heads (groups of 8); reported beside the main step.
LONG_GQA = Workload("bwd_bf16_b1_h16_hkv2_n16384_d128", "bf16", 1, 16, 16384, 128, (False, True), True, 1007, Hkv=2)


# The kernel benchmark grid of that section: 16k tokens per batch with
# H * d = 2048, sequence lengths 512 .. 16384 (B = 16384 / N), head dims 64
# (32 heads) and 128 (16 heads), both masks. Timed in the benchmark's report,
# forward and backward, on inputs drawn on the device (timing only: the
# outputs are not compared there; parity at these shapes is the tests').
SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP_D = (64, 128)
SWEEP_TOKENS = 16384
SWEEP_HIDDEN = 2048


def sweep_shape(N: int, d: int):
    """(B, H, N, d) of the sweep point with sequence length N and head dim d."""
    return SWEEP_TOKENS // N, SWEEP_HIDDEN // d, N, d


def make_qkv_device(B: int, H: int, N: int, d: int, seed: int, device, with_do: bool = True):
    """Q, K, V (and dO) [B, N, H, d] drawn on `device` by a generator seeded there: randn float32 rounded to
    bfloat16, in that order. For timing runs whose outputs nothing compares (drawing the largest shapes on
    the CPU takes seconds)."""
    g = torch.Generator(device=device).manual_seed(seed)
    n = 4 if with_do else 3
    return tuple(torch.randn(B, N, H, d, dtype=torch.float32, generator=g, device=device).to(torch.bfloat16)
                 for _ in range(n))


@dataclass(frozen=True)
class DecodeWorkload:
    """Decoding: Nq new query rows per sequence against a cache of Nk keys and values."""
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: tuple
    seed: int

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())


# Token-by-token generation against a 16k-token cache (the longest context of
# the sweep above): 16 sequences, 32 query heads in groups of 4 per K/V head,
# one new token each (the causal mask then hides nothing); and 4 new tokens
# at once under the causal mask. The pages describe no decoding workload;
# these are the plainest shapes that keep the cache at 16k tokens and H * d at
# 4096 query features.
DECODE_1 = DecodeWorkload("decode_bf16_b16_h32_hkv8_nq1_nk16384_d128", 16, 32, 8, 1, 16384, 128, (False,), 1008)
DECODE_4 = DecodeWorkload("decode_bf16_b16_h32_hkv8_nq4_nk16384_d128", 16, 32, 8, 4, 16384, 128, (True,), 1009)


def make_decode(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int = 0):
    """Decoding inputs on the CPU: Q [B, Nq, H, d], then K and V [B, Nk, Hkv, d], drawn in that order
    from one generator (randn, float32, rounded to bfloat16)."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for n, h in ((Nq, H), (Nk, Hkv), (Nk, Hkv)):
        out.append(torch.randn(B, n, h, d, dtype=torch.float32, generator=g).to(torch.bfloat16))
    return tuple(out)


def make_fp8(B: int, H: int, N: int, d: int, seed: int = 0):
    """FP8 inputs on the CPU: Q, K, V drawn as make_qkv draws them (randn float32), each quantised per tensor
    to E4M3 with descale = amax / 448 (rounded to fp32) by torch's float8_e4m3fn conversion (nearest even).
    Returns (q8, k8, v8 [B, N, H, d] float8_e4m3fn, vt8 [B, H, d, ldv] uint8 with zero padding,
    (q_descale, k_descale, v_descale))."""
    g = torch.Generator().manual_seed(seed)
    out, ds = [], []
    for _ in range(3):
        x = torch.randn(B, N, H, d, dtype=torch.float32, generator=g)
        s = float(torch.tensor(float(x.abs().max()) / 448.0, dtype=torch.float32))
        out.append((x / s).to(torch.float8_e4m3fn))
        ds.append(s)
    ldv = (N + 63) // 64 * 64
    vt8 = torch.zeros(B, H, d, ldv, dtype=torch.uint8)
    vt8[..., :N] = out[2].view(torch.uint8).permute(0, 2, 3, 1)
    return out[0], out[1], out[2], vt8.contiguous(), tuple(ds)


# The FP8 forward at the long-context shape (reported beside the bf16 step).
FP8_LONG = Workload("fwd_fp8_b1_h16_n16384_d128", "fp8", 1, 16, 16384, 128, (False, True), False, 1010)


def make_qkv(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0, with_do: bool = False):
    """Draw Q, K, V (and dO) on the CPU. Returns a tuple of CPU tensors [B, N, H, d].

    dtype "bf16" rounds the float32 draws to bfloat16 (RNE); "fp32" keeps them.
    """
    g = torch.Generator().manual_seed(seed)
    n = 4 if with_do else 3
    out = []
    for _ in range(n):
        t = torch.randn(B, N, H, d, dtype=torch.float32, generator=g)
        out.append(t.to(torch.bfloat16) if dtype == "bf16" else t)
    return tuple(out)


def make_gqa(B: int, H: int, Hkv: int, N: int, d: int, dtype: str = "bf16", seed: int = 0, with_do: bool = False):
    """Grouped-query inputs: Q [B, N, H, d], then K and V [B, N, Hkv, d] (and dO [B, N, H, d]), drawn in that
    order from one generator, as make_qkv does."""
    g = torch.Generator().manual_seed(seed)
    heads = [H, Hkv, Hkv] + ([H] if with_do else [])
    out = []
    for h in heads:
        t = torch.randn(B, N, h, d, dtype=torch.float32, generator=g)
        out.append(t.to(torch.bfloat16) if dtype == "bf16" else t)
    return tuple(out)


def make_workload(w: Workload):
    """Inputs of a named workload: (q, k, v) or (q, k, v, do) on the CPU."""
    if w.Hkv and w.Hkv != w.H:
        return make_gqa(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed, with_do=w.backward)
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, with_do=w.backward)
