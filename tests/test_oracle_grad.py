"""Pins for the fp64 backward oracle (CPU only).

The pages only say that gradients, like outputs, are compared within a
numerical tolerance (page "FlashAttention-2: atención eficiente en GPU para
contextos largos", section "Bloques pequeños, normalización global"). The
analytic backward in :mod:`oracle.attn_ref` is pinned here by the hand-derived
fixture, central finite differences of the (independently pinned) forward,
torch's CPU fp64 autograd through its own attention routine, and identities
that any correct gradient satisfies.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attn_bwd, attn_bwd_head, attn_fwd, attn_fwd_head

from test_oracle import load_golden


@pytest.mark.parametrize("mask", ["noncausal", "causal"])
def test_golden_backward(golden_dir, mask):
    g = load_golden(golden_dir, "hand_n2_d1.json")
    dq, dk, dv = attn_bwd(g["q"], g["k"], g["v"], g["do"], mask == "causal", g["scale"])
    exp = g["expected"][mask]
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(got.reshape(-1), exp[name], rtol=0, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 2), (3, 2), (5, 3)])
def test_finite_differences(causal, N, d):
    """dL/dX for L = sum(dO * O(Q, K, V)), by central differences with h = 1e-6."""
    rng = np.random.default_rng(N * 13 + d + 7 * causal)
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    s = 0.6
    g = attn_bwd_head(q, k, v, do, causal, s)

    def loss(q_, k_, v_):
        return float((attn_fwd_head(q_, k_, v_, causal, s)[0] * do).sum())

    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("N,d", [(17, 8), (96, 64), (160, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd(N, d, causal):
    gen = torch.Generator().manual_seed(N + d + causal)
    B, H = 2, 2
    q, k, v, do = (torch.randn(B, N, H, d, dtype=torch.float64, generator=gen) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = attn_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), causal, scale)
    qt, kt, vt = (x.permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    o.backward(do.permute(0, 2, 1, 3))
    for name, got, ref in (("dq", dq, qt.grad), ("dk", dk, kt.grad), ("dv", dv, vt.grad)):
        np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-10, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    rng = np.random.default_rng(12)
    N, d = 70, 16
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    g = attn_bwd_head(q, k, v, do, causal, 0.25)
    np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, rtol=0, atol=1e-10)
    o, lse = attn_fwd_head(q, k, v, causal, 0.25)
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["lse"], lse, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["D"], (do * o).sum(axis=1), rtol=0, atol=1e-10)
    assert abs((g["dq"] * q).sum() - (g["dk"] * k).sum()) < 1e-10


def test_backward_row_chunks():
    """More than one row chunk: the chunked accumulation of dK, dV matches torch autograd."""
    gen = torch.Generator().manual_seed(77)
    N, d = 1300, 16
    q, k, v, do = (torch.randn(1, N, 1, d, dtype=torch.float64, generator=gen) for _ in range(4))
    dq, dk, dv = attn_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), True, 0.25)
    qt, kt, vt = (x.permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
    o.backward(do.permute(0, 2, 1, 3))
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-10)


def test_forward_backward_agree_on_o_and_lse():
    rng = np.random.default_rng(13)
    B, N, H, d = 1, 40, 2, 8
    q, k, v, do = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    o, lse = attn_fwd(q, k, v, True, 0.5)
    g = attn_bwd_head(q[0, :, 1], k[0, :, 1], v[0, :, 1], do[0, :, 1], True, 0.5)
    np.testing.assert_allclose(g["o"], o[0, :, 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["lse"], lse[0, 1], rtol=0, atol=1e-13)
