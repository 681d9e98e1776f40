"""Decoding against a key/value cache, and the split-KV combination of partial results.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

Source: page "FlashAttention-2: atención eficiente en GPU para contextos
largos", section "Cómo documentar una diferencia técnica": the initial pass
over the context (prefill) and token-by-token generation (decoding) are to be
told apart, because their bottlenecks can differ. The page gives no algorithm
for decoding. Readings used here:

* Decoding computes the same exact attention as :mod:`oracle.attn_ref`, for a
  few new query rows against a cache of ``Nk`` keys and values. Q, O are
  ``[B, Nq, H, d]``; K, V ``[B, Nk, Hkv, d]`` with query head h reading K/V
  head h // (H / Hkv) as in :mod:`oracle.gqa`; LSE ``[B, H, Nq]``.
* Query row i is the token at position ``Nk - Nq + i`` of the sequence (the
  new tokens are the last ``Nq`` positions, their own keys already appended to
  the cache). Under the causal mask it sees keys ``j <= Nk - Nq + i``; with
  ``Nq = Nk`` this is the causal mask of :mod:`oracle.attn_ref`.
* Split-KV: the key range is cut into chunks; each chunk gives, per query row,
  the attention restricted to its keys, ``O_s`` (normalised within the chunk)
  and ``LSE_s`` (its log-sum-exp; ``-inf`` and ``O_s = 0`` when the chunk holds
  no visible key for that row). The exact result follows from the softmax
  algebra the same page's section "Bloques pequeños, normalización global"
  relies on (a global normaliser from per-block statistics):

      LSE = ln sum_s exp(LSE_s),     O = sum_s exp(LSE_s - LSE) O_s.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _group(H: int, Hkv: int) -> int:
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"H = {H} is not a multiple of Hkv = {Hkv}")
    return H // Hkv


def _scores(qh: np.ndarray, kh: np.ndarray, causal: bool, scale: float, kbeg: int, kend: int) -> np.ndarray:
    """Scaled, masked scores [Nq, kend - kbeg] of one head's query rows against keys kbeg .. kend-1."""
    nq, nk = qh.shape[0], kh.shape[0]
    s = scale * (qh @ kh[kbeg:kend].T)
    if causal:
        pos = nk - nq + np.arange(nq)                 # sequence position of each query row
        keys = np.arange(kbeg, kend)
        s = np.where(keys[None, :] <= pos[:, None], s, -np.inf)
    return s


def attn_partial(q, k, v, causal: bool, scale: float, kbeg: int, kend: int):
    """Attention of every query row restricted to keys kbeg .. kend-1.

    Returns (O_s [B, Nq, H, d], LSE_s [B, H, Nq]); a row with no visible key
    in the range gets O_s = 0 and LSE_s = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, H, _ = q.shape
    G = _group(H, k.shape[2])
    if not (0 <= kbeg <= kend <= k.shape[1]):
        raise ValueError("key range out of bounds")
    o = np.zeros((B, nq, H, v.shape[3]))
    lse = np.full((B, H, nq), -np.inf)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, :, h], k[b, :, h // G], causal, scale, kbeg, kend)
            if s.shape[1] == 0:
                continue
            m = s.max(axis=1)
            live = np.isfinite(m)
            e = np.exp(s[live] - m[live, None])
            l = e.sum(axis=1)
            o[b, live, h] = (e / l[:, None]) @ v[b, kbeg:kend, h // G]
            lse[b, h, live] = m[live] + np.log(l)
    return o, lse


def attn_decode(q, k, v, causal: bool, scale: float):
    """Exact attention of the Nq query rows against the whole cache: (O [B, Nq, H, d], LSE [B, H, Nq])."""
    q, k = _f64(q), _f64(k)
    if causal and q.shape[1] > k.shape[1]:
        raise ValueError("causal decoding needs Nq <= Nk")
    return attn_partial(q, k, v, causal, scale, 0, k.shape[1])


def merge_partials(o_parts, lse_parts):
    """Combine per-chunk results (lists of O_s [B, Nq, H, d] and LSE_s [B, H, Nq]) into (O, LSE)."""
    lse_s = np.stack([_f64(x) for x in lse_parts])          # [S, B, H, Nq]
    o_s = np.stack([_f64(x) for x in o_parts])              # [S, B, Nq, H, d]
    mx = lse_s.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse_s - safe[None])                          # exp(LSE_s - max); 0 for empty chunks
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    coef = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)   # exp(LSE_s - LSE)
    o = np.einsum("sbhn,sbnhd->bnhd", coef, o_s)
    return o, lse


def attn_decode_split(q, k, v, causal: bool, scale: float, bounds):
    """Split-KV decoding: partial attention over each (kbeg, kend) chunk of ``bounds``, then merge."""
    parts = [attn_partial(q, k, v, causal, scale, b0, b1) for b0, b1 in bounds]
    return merge_partials([p[0] for p in parts], [p[1] for p in parts])


def bytes_decode(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> float:
    """Compulsory HBM bytes of one bf16 decode call: read K and V (the cache) and Q, write O and LSE."""
    return 2.0 * (2 * B * Nk * Hkv * d) + 2.0 * (2 * B * Nq * H * d) + 4.0 * B * H * Nq
