"""Tile-by-tile online-softmax forward in fp64, and its negative control.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`). This is the algorithm the pages
describe, written from their description so that tests can show it reaches
the plain definition in :mod:`oracle.attn_ref`:

* page "FlashAttention-2: atención eficiente en GPU para contextos largos",
  section "Bloques pequeños, normalización global": the inputs are split into
  blocks processed in fast on-chip memory; an online softmax keeps running
  row statistics and rescales the partial output so that the result stays
  normalised over the whole row; normalising each block on its own and adding
  the results is a different computation (:func:`blockwise_normalised_sum`);
* same page, section "Tres mejoras en la utilización de la GPU": part of the
  rescaling and of the boundary and causal-mask handling is removed from the
  inner loop. Here that means: key blocks entirely above the diagonal are
  never visited, the mask is applied only to blocks that straddle the
  diagonal or the ragged tail, and the division by the row sum happens once
  at the end.

Per query block (rows r, of at most Br) and key block j (of at most Bc):

    S    = scale * Q_r K_j^T                 (masked only where needed)
    m'   = max(m, rowmax(S))
    a    = exp(m - m')                       (rescale of the running state)
    Pt   = exp(S - m')
    l    = a * l + rowsum(Pt)
    acc  = a * acc + Pt V_j
    m    = m'
  finally  O_r = acc / l,  LSE_r = m + ln l.
"""

from __future__ import annotations

import numpy as np


def online_fwd_head(q, k, v, causal: bool, scale: float, br: int, bc: int):
    """Online-softmax forward for one (b, h): q, k, v [N, d] -> (O [N, d], LSE [N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for r0 in range(0, n, br):
        r1 = min(n, r0 + br)
        rows = np.arange(r0, r1)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, v.shape[1]))
        # Causal: key blocks that start after the last query row are skipped.
        k_end = min(n, r1) if causal else n
        for c0 in range(0, k_end, bc):
            c1 = min(k_end, c0 + bc)
            cols = np.arange(c0, c1)
            s = scale * (q[r0:r1] @ k[c0:c1].T)
            straddles = causal and c1 - 1 > r0
            if straddles:
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - m_new)  # exp(-inf) = 0 on the first visited block
            pt = np.exp(s - m_new[:, None])
            l = alpha * l + pt.sum(axis=1)
            acc = alpha[:, None] * acc + pt @ v[c0:c1]
            m = m_new
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def blockwise_normalised_sum(q, k, v, scale: float, bc: int):
    """Negative control: softmax each key block on its own and add the block outputs.

    The pages state that this is not the same computation as attention over
    the whole row; tests check that it differs from the definition.
    Non-causal only; q, k, v [N, d] -> O [N, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    out = np.zeros((q.shape[0], v.shape[1]))
    for c0 in range(0, n, bc):
        s = scale * (q @ k[c0:c0 + bc].T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out += (e / e.sum(axis=1, keepdims=True)) @ v[c0:c0 + bc]
    return out
