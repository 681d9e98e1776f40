"""Pins for the fp64 forward oracle (CPU only).

Each test checks :mod:`oracle` against something other than itself: the
hand-derived fixtures in ``tests/golden``, scalar brute force written by a
different algebraic route, torch's CPU fp64 library routines, closed forms,
invariants, and the pages' own statement that the tiled online softmax is the
same computation while per-block normalisation is not (page
"FlashAttention-2: atención eficiente en GPU para contextos largos", section
"Bloques pequeños, normalización global").
"""

import ast
import json
import math
import operator
import os

import numpy as np
import pytest
import torch

from oracle import attn_fwd, attn_fwd_head, attn_fwd_rows
from oracle.brute import brute_fwd
from oracle.online import blockwise_normalised_sum, online_fwd_head

# ---------------------------------------------------------------------------
# Golden fixtures: exact expressions evaluated by a restricted parser.

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg}


def _ev(expr: str) -> float:
    def go(n):
        if isinstance(n, ast.Expression):
            return go(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.BinOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](go(n.left), go(n.right))
        if isinstance(n, ast.UnaryOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](go(n.operand))
        if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "ln" and len(n.args) == 1:
            return math.log(go(n.args[0]))
        raise ValueError(f"unsupported expression {expr!r}")
    return go(ast.parse(expr, mode="eval"))


def _arr(x):
    if isinstance(x, str):
        return _ev(x)
    return [_arr(e) for e in x]


def load_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)
    s = g["shape"]
    B, N, H, d = s["B"], s["N"], s["H"], s["d"]

    def t(key):
        a = np.array(_arr(g[key]), dtype=np.float64)
        return a.reshape(B, N, H, -1)
    out = {"scale": _ev(g["scale"]), "q": t("q"), "k": t("k"), "v": t("v"), "expected": {}}
    if "do" in g:
        out["do"] = t("do")
    for mask, e in g["expected"].items():
        out["expected"][mask] = {key: np.array(_arr(val), dtype=np.float64) for key, val in e.items()}
    return out


@pytest.mark.parametrize("name", ["hand_n2_d1.json", "hand_n3_d2.json"])
@pytest.mark.parametrize("mask", ["noncausal", "causal"])
def test_golden_forward(golden_dir, name, mask):
    g = load_golden(golden_dir, name)
    o, lse = attn_fwd(g["q"], g["k"], g["v"], mask == "causal", g["scale"])
    exp = g["expected"][mask]
    np.testing.assert_allclose(o.reshape(exp["o"].shape), exp["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse.reshape(exp["lse"].shape), exp["lse"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Brute force (scalar loops, no max subtraction, P_ij = 1 / sum_k exp(S_ik - S_ij)).

@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(N, d, causal):
    rng = np.random.default_rng(100 * N + 10 * d + causal)
    B, H = 2, 2
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    scale = 0.7
    o, lse = attn_fwd(q, k, v, causal, scale)
    ob, lseb = brute_fwd(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Library cross-check: torch CPU fp64 scaled_dot_product_attention and logsumexp.

@pytest.mark.parametrize("N,d", [(17, 8), (64, 64), (200, 32), (256, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa_forward(N, d, causal):
    g = torch.Generator().manual_seed(N * 7 + d + causal)
    B, H = 2, 3
    q, k, v = (torch.randn(B, N, H, d, dtype=torch.float64, generator=g) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q.numpy(), k.numpy(), v.numpy(), causal, scale)
    qt, kt, vt = (x.permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-10)
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# Closed forms.

def test_probability_rows_sum_to_one():
    """With V = identity (d_v = N), O is P itself: rows are non-negative and sum to 1."""
    rng = np.random.default_rng(3)
    N, d = 37, 16
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    for causal in (False, True):
        p, _ = attn_fwd_head(q, k, np.eye(N), causal, 0.25)
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    rng = np.random.default_rng(4)
    N, d = 50, 8
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    row = rng.standard_normal(d)
    o, _ = attn_fwd_head(q, k, np.tile(row, (N, 1)), causal, 0.5)
    np.testing.assert_allclose(o, np.tile(row, (N, 1)), rtol=0, atol=1e-12)


def test_causal_row0():
    rng = np.random.default_rng(5)
    N, d = 40, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = attn_fwd_head(q, k, v, True, 0.3)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_attention(causal):
    """Q = 0: every visible key has the same score, so O is a (prefix) mean of V."""
    rng = np.random.default_rng(6)
    N, d = 33, 4
    k, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    o, lse = attn_fwd_head(np.zeros((N, d)), k, v, causal, 1.0)
    if causal:
        cnt = np.arange(1, N + 1)
        np.testing.assert_allclose(o, np.cumsum(v, axis=0) / cnt[:, None], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-13)
    else:
        np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (N, 1)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.full(N, math.log(N)), rtol=0, atol=1e-13)


def test_single_token():
    q, k, v = np.array([[1.0, -2.0]]), np.array([[0.5, 3.0]]), np.array([[7.0, -1.0]])
    for causal in (False, True):
        o, lse = attn_fwd_head(q, k, v, causal, 0.5)
        np.testing.assert_allclose(o, v, rtol=0, atol=0)
        assert lse[0] == pytest.approx(0.5 * (0.5 - 6.0), abs=1e-15)


# ---------------------------------------------------------------------------
# Invariants.

@pytest.mark.parametrize("causal", [False, True])
def test_key_translation(causal):
    """K -> K + c (every row) leaves O unchanged and shifts LSE_i by scale * q_i . c."""
    rng = np.random.default_rng(7)
    N, d, s = 45, 8, 0.4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    c = rng.standard_normal(d)
    o1, l1 = attn_fwd_head(q, k, v, causal, s)
    o2, l2 = attn_fwd_head(q, k + c, v, causal, s)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + s * (q @ c), rtol=0, atol=1e-12)


def test_permutation_noncausal():
    rng = np.random.default_rng(8)
    N, d = 30, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = attn_fwd_head(q, k, v, False, 0.5)
    pk, pq = rng.permutation(N), rng.permutation(N)
    o2, lse2 = attn_fwd_head(q[pq], k[pk], v[pk], False, 0.5)
    np.testing.assert_allclose(o2, o[pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse[pq], rtol=0, atol=1e-12)


def test_large_scores_stay_finite():
    """Scores of order 1e4: P is (near) one-hot, O is the V row of the arg-max key."""
    rng = np.random.default_rng(9)
    N, d = 20, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    q, k = 100 * q, 100 * k
    for causal in (False, True):
        o, lse = attn_fwd_head(q, k, v, causal, 1.0)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        s = q @ k.T
        if causal:
            s = np.where(np.tril(np.ones((N, N))) > 0, s, -np.inf)
        idx = s.argmax(axis=1)
        np.testing.assert_allclose(o, v[idx], rtol=0, atol=1e-6)
        np.testing.assert_allclose(lse, s.max(axis=1), rtol=1e-12, atol=1e-6)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    N, d = 2100, 16  # more than one row chunk
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = attn_fwd_head(q, k, v, causal, 0.25)
        rows = np.array([0, 1, 1023, 1024, 1500, 2099])
        o2, l2 = attn_fwd_rows(q, k, v, rows, causal, 0.25)
        np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, lse[rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# The tiled online softmax reaches the definition; per-block normalisation does not.

@pytest.mark.parametrize("br", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("bc", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_online_rewrite_matches(br, bc, causal):
    rng = np.random.default_rng(br * 31 + bc)
    N, d = 37, 8  # no tile size divides N
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = attn_fwd_head(q, k, v, causal, 0.35)
    o2, l2 = online_fwd_head(q, k, v, causal, 0.35, br, bc)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_blockwise_normalisation_is_not_attention():
    rng = np.random.default_rng(11)
    N, d = 64, 16
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, _ = attn_fwd_head(q, k, v, False, 0.25)
    wrong = blockwise_normalised_sum(q, k, v, 0.25, 16)
    assert np.abs(wrong - o).max() > 1e-2
    # With a single block covering every key it coincides with attention.
    np.testing.assert_allclose(blockwise_normalised_sum(q, k, v, 0.25, N), o, rtol=0, atol=1e-12)
