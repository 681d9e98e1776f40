"""Plain fp64 definition of exact softmax attention and its gradients.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`). Nothing here is tiled, fused or
reordered beyond the definition: each query row's scores against all visible
keys are formed, normalised by a row softmax and contracted with V. Rows are
independent, so processing query rows in chunks of at most ``MAX_ROWS`` is
still the naive definition (it only bounds memory).

Definition (page "FlashAttention-2: atención eficiente en GPU para contextos
largos", section "El coste de mover datos en secuencias largas": the
conventional computation forms the full score matrix and the full probability
matrix; the same page's section "Bloques pequeños, normalización global"
states that the tiled method computes exactly this attention):

    S   = scale * Q K^T                       (N x N per batch b, head h)
    S_ij = -inf  for j > i                    (causal variant only)
    m_i = max_j S_ij,   l_i = sum_j exp(S_ij - m_i)
    P_ij = exp(S_ij - m_i) / l_i
    O   = P V,          LSE_i = m_i + ln l_i  (natural log)

Readings where the pages are silent:

* causal: key j is visible to query i iff j <= i (query and key sequences
  have the same length, so top-left and bottom-right alignment coincide);
* ``scale`` is applied to Q K^T before masking and softmax, and is used as the
  caller passes it (the HIP path receives an fp32 value; pass that same value,
  widened to fp64, here);
* LSE is the natural-log log-sum-exp of the scaled, masked scores.

Backward (the pages only say that gradients are checked within a tolerance,
in section "Bloques pequeños, normalización global"; this is the textbook
chain rule through the row softmax, for upstream gradient dO = dL/dO):

    dV   = P^T dO
    dP   = dO V^T
    D_i  = sum_j P_ij dP_ij            (= dO_i . O_i)
    dS   = P o (dP - D 1^T)
    dQ   = scale * dS K
    dK   = scale * dS^T Q

Masked entries have P = 0 and hence dS = 0.

Tensor layout: Q, K, V, O, dO, dQ, dK, dV are ``[B, N, H, d]`` (d fastest);
LSE and D are ``[B, H, N]``. All inputs are converted to float64.
"""

from __future__ import annotations

import numpy as np

MAX_ROWS = 1024


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, causal: bool, scale: float):
    """Scaled, masked scores of the given query rows against all keys: [len(rows), N]."""
    s = scale * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax of scores with -inf entries; returns (P, m, l)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def attn_fwd_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, causal: bool, scale: float):
    """Attention output and LSE for selected query rows of one (batch, head).

    q, k, v: [N, d] for one (b, h). rows: 1-D integer array of query indices.
    Returns (O[rows] as [len(rows), d], LSE[rows] as [len(rows)]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, MAX_ROWS):
        r = rows[c0:c0 + MAX_ROWS]
        p, m, l = _softmax_rows(_scores(q[r], k, r, causal, scale))
        o[c0:c0 + r.size] = p @ v
        lse[c0:c0 + r.size] = m + np.log(l)
    return o, lse


def attn_fwd_head(q, k, v, causal: bool, scale: float):
    """Forward for one (b, h): q, k, v [N, d] -> (O [N, d], LSE [N])."""
    return attn_fwd_rows(q, k, v, np.arange(np.shape(q)[0]), causal, scale)


def attn_fwd(q, k, v, causal: bool, scale: float):
    """Forward over all (b, h): q, k, v [B, N, H, d] -> (O [B, N, H, d], LSE [B, H, N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, d = q.shape
    o = np.empty((B, N, H, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h, :], lse[b, h, :] = attn_fwd_head(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :],
                                                         causal, scale)
    return o, lse


def attn_bwd_head(q, k, v, do, causal: bool, scale: float):
    """Gradients for one (b, h) from its own fp64 forward.

    q, k, v, do: [N, d]. Returns dict with dq, dk, dv [N, d] and o [N, d],
    lse [N], D [N] (D_i = sum_j P_ij dP_ij).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    N = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.empty_like(v)
    lse = np.empty(N)
    dd = np.empty(N)
    for r0 in range(0, N, MAX_ROWS):
        r = np.arange(r0, min(N, r0 + MAX_ROWS))
        p, m, l = _softmax_rows(_scores(q[r], k, r, causal, scale))
        o[r] = p @ v
        lse[r] = m + np.log(l)
        dv += p.T @ do[r]
        dp = do[r] @ v.T
        di = (p * dp).sum(axis=1)
        dd[r] = di
        ds = p * (dp - di[:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "D": dd}


def attn_bwd(q, k, v, do, causal: bool, scale: float):
    """Gradients over all (b, h): inputs [B, N, H, d] -> (dq, dk, dv) [B, N, H, d]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, H, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            g = attn_bwd_head(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :], causal, scale)
            dq[b, :, h, :], dk[b, :, h, :], dv[b, :, h, :] = g["dq"], g["dk"], g["dv"]
    return dq, dk, dv
