"""Scalar-loop brute force for tiny attention problems.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`). Used solely to pin
:mod:`oracle.attn_ref`, so it takes a different algebraic route on purpose:
no max subtraction and no matrix products. Each probability is formed as

    P_ij = 1 / sum_{k visible} exp(S_ik - S_ij)

which equals exp(S_ij) / sum_k exp(S_ik), and the log-sum-exp is
``log(fsum(exp(S_ik)))`` taken directly. Both are fine for the small score
magnitudes the tests use. Inputs are nested Python lists or arrays
[B][N][H][d]; outputs are nested lists.
"""

from __future__ import annotations

import math


def brute_fwd(q, k, v, causal: bool, scale: float):
    """Returns (O as [B][N][H][d] lists, LSE as [B][H][N] lists)."""
    B = len(q)
    N = len(q[0])
    H = len(q[0][0])
    d = len(q[0][0][0])
    dv = len(v[0][0][0])
    o = [[[[0.0] * dv for _ in range(H)] for _ in range(N)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                visible = [j for j in range(N) if (not causal) or j <= i]
                s = {}
                for j in visible:
                    s[j] = scale * math.fsum(float(q[b][i][h][c]) * float(k[b][j][h][c]) for c in range(d))
                lse[b][h][i] = math.log(math.fsum(math.exp(s[j]) for j in visible))
                for j in visible:
                    pij = 1.0 / math.fsum(math.exp(s[t] - s[j]) for t in visible)
                    for c in range(dv):
                        o[b][i][h][c] += pij * float(v[b][j][h][c])
    return o, lse
