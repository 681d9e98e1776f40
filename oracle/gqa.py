"""Grouped-query (and multi-query) attention: plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

Source: page "FlashAttention-T: Optimización GPU para LLMs Escalables",
section "Innovaciones técnicas frente a FlashAttention original": the
backward pass supports multi-query and grouped-query attention natively. The
page does not define them; the reading used here is the standard one. Q has H
heads, K and V have Hkv heads with H a multiple of Hkv; query head h attends
with K/V head h // G, G = H / Hkv (G = H is multi-query attention, G = 1 is
ordinary multi-head attention). Each query head is exactly the attention of
:mod:`oracle.attn_ref` on its K/V head. A K/V head receives, as its gradient,
the sum of the gradients of the G query heads that read it (the chain rule
through the shared operand).

Tensor layout: Q, O, dO, dQ ``[B, N, H, d]``; K, V, dK, dV ``[B, N, Hkv, d]``;
LSE ``[B, H, N]``.
"""

from __future__ import annotations

import numpy as np

from .attn_ref import attn_bwd_head, attn_fwd_head


def _group(H: int, Hkv: int) -> int:
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"H = {H} is not a multiple of Hkv = {Hkv}")
    return H // Hkv


def attn_fwd_gqa(q, k, v, causal: bool, scale: float):
    """q [B, N, H, d], k, v [B, N, Hkv, d] -> (O [B, N, H, d], LSE [B, H, N])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, N, H, d = q.shape
    G = _group(H, k.shape[2])
    o = np.empty((B, N, H, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, :, h], lse[b, h] = attn_fwd_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G], causal, scale)
    return o, lse


def attn_bwd_gqa(q, k, v, do, causal: bool, scale: float):
    """Gradients: dq [B, N, H, d]; dk, dv [B, N, Hkv, d] summed over each group."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, N, H, d = q.shape
    G = _group(H, k.shape[2])
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = attn_bwd_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G], do[b, :, h], causal, scale)
            dq[b, :, h] = g["dq"]
            dk[b, :, h // G] += g["dk"]
            dv[b, :, h // G] += g["dv"]
    return dq, dk, dv
