"""Pins of the grouped-query / multi-query oracle (oracle.gqa) against things
other than itself: torch CPU fp64 scaled_dot_product_attention with
enable_gqa and its autograd (independent library code), the reduction to the
multi-head oracle when every query head has its own K/V head, and central
finite differences of L = sum(dO * O) with respect to a shared K/V head
(which checks that a shared head's gradient sums its whole group)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn_bwd, attn_bwd_gqa, attn_fwd, attn_fwd_gqa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_ref(q, k, v, do, causal, scale):
    # [B, N, H, d] -> [B, H, N, d]
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
    G = q.shape[2] // k.shape[2]
    s = scale * torch.einsum("bhnd,bhmd->bhnm", tq.detach(), tk.detach().repeat_interleave(G, dim=1))
    if causal:
        n = q.shape[1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    t = lambda x: x.detach().numpy().transpose(0, 2, 1, 3)
    return t(o), lse.numpy(), t(tq.grad), t(tk.grad), t(tv.grad)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (6, 2), (4, 4)])
@pytest.mark.parametrize("N", [1, 5, 17])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_torch_sdpa(H, Hkv, N, causal):
    B, d = 2, 8
    q, do = _rand((B, N, H, d), 1), _rand((B, N, H, d), 2)
    k, v = _rand((B, N, Hkv, d), 3), _rand((B, N, Hkv, d), 4)
    scale = 0.37
    ro, rl, rq, rk, rv = _torch_ref(q, k, v, do, causal, scale)
    o, lse = attn_fwd_gqa(q, k, v, causal, scale)
    dq, dk, dv = attn_bwd_gqa(q, k, v, do, causal, scale)
    for got, ref in ((o, ro), (lse, rl), (dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_with_one_kv_head_per_query_head_is_mha(causal):
    q, k, v, do = (_rand((2, 9, 3, 4), s) for s in (5, 6, 7, 8))
    o1, l1 = attn_fwd_gqa(q, k, v, causal, 0.5)
    o2, l2 = attn_fwd(q, k, v, causal, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for a, b in zip(attn_bwd_gqa(q, k, v, do, causal, 0.5), attn_bwd(q, k, v, do, causal, 0.5)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_shared_head_gradient_finite_differences(causal):
    B, N, H, Hkv, d = 1, 4, 3, 1, 3
    q, do = _rand((B, N, H, d), 9), _rand((B, N, H, d), 10)
    k, v = _rand((B, N, Hkv, d), 11), _rand((B, N, Hkv, d), 12)
    scale, h = 0.8, 1e-6
    loss = lambda q_, k_, v_: float((attn_fwd_gqa(q_, k_, v_, causal, scale)[0] * do).sum())
    dq, dk, dv = attn_bwd_gqa(q, k, v, do, causal, scale)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args = {"q": q, "k": k, "v": v}
            fp = loss(*(xp if n == name else args[n] for n in "qkv"))
            fm = loss(*(xm if n == name else args[n] for n in "qkv"))
            assert abs((fp - fm) / (2 * h) - g[i]) <= 1e-6 * max(1.0, abs(g[i])), (name, i)


def test_gqa_rejects_head_counts_that_do_not_divide():
    q = np.zeros((1, 2, 4, 2))
    kv = np.zeros((1, 2, 3, 2))
    with pytest.raises(ValueError):
        attn_fwd_gqa(q, kv, kv, False, 1.0)
