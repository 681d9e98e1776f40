"""Pins of the decoding oracle (oracle.decode) against things other than itself:

* a hand-derived fixture (tests/golden/hand_decode_nq2_nk3_d2.json) with the
  full result and the two split-KV partials as exact expressions;
* torch CPU fp64 scaled_dot_product_attention with an explicit boolean mask
  built for bottom-right alignment, K/V heads repeated per group, and
  torch.logsumexp for LSE (independent library code);
* the reduction to the prefill oracle when Nq = Nk, and the last Nq rows of
  a causal prefill (decoding the newest tokens of a sequence gives the same
  rows as processing the whole sequence);
* split-and-merge against the unsplit result for single, even, ragged and
  fully-masked chunks, plus identities of the merge itself.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn_fwd_gqa
from oracle.decode import attn_decode, attn_decode_split, attn_partial, bytes_decode, merge_partials
from test_oracle import _arr


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _golden(golden_dir):
    import json
    import os

    with open(os.path.join(golden_dir, "hand_decode_nq2_nk3_d2.json")) as f:
        g = json.load(f)
    s = g["shape"]
    q = np.array(_arr(g["q"])).reshape(s["B"], s["Nq"], s["H"], s["d"])
    k = np.array(_arr(g["k"])).reshape(s["B"], s["Nk"], s["Hkv"], s["d"])
    v = np.array(_arr(g["v"])).reshape(s["B"], s["Nk"], s["Hkv"], s["d"])
    return g, q, k, v, float(_arr(g["scale"]))


@pytest.mark.parametrize("mask", ["noncausal", "causal"])
def test_golden_decode(golden_dir, mask):
    g, q, k, v, scale = _golden(golden_dir)
    o, lse = attn_decode(q, k, v, mask == "causal", scale)
    e = g["expected"][mask]
    assert np.allclose(o[0, :, 0], np.array(_arr(e["o"])), rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], np.array(_arr(e["lse"])), rtol=0, atol=1e-12)


def test_golden_decode_chunks_and_merge(golden_dir):
    g, q, k, v, scale = _golden(golden_dir)
    parts = []
    for c in g["expected"]["causal_chunks"]:
        o, lse = attn_partial(q, k, v, True, scale, c["kbeg"], c["kend"])
        assert np.allclose(o[0, :, 0], np.array(_arr(c["o"])), rtol=0, atol=1e-12)
        assert np.allclose(lse[0, 0], np.array(_arr(c["lse"])), rtol=0, atol=1e-12)
        parts.append((o, lse))
    o, lse = merge_partials([p[0] for p in parts], [p[1] for p in parts])
    e = g["expected"]["causal"]
    assert np.allclose(o[0, :, 0], np.array(_arr(e["o"])), rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], np.array(_arr(e["lse"])), rtol=0, atol=1e-12)


def _torch_decode(q, k, v, causal, scale):
    # [B, N, H, d] -> [B, H, N, d]; K/V heads repeated so every query head has its own
    G = q.shape[2] // k.shape[2]
    tq = torch.tensor(q.transpose(0, 2, 1, 3), dtype=torch.float64)
    tk = torch.tensor(k.transpose(0, 2, 1, 3), dtype=torch.float64).repeat_interleave(G, dim=1)
    tv = torch.tensor(v.transpose(0, 2, 1, 3), dtype=torch.float64).repeat_interleave(G, dim=1)
    nq, nk = q.shape[1], k.shape[1]
    allowed = None
    if causal:
        allowed = torch.tensor(np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None])
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(~allowed, float("-inf"))
    return o.numpy().transpose(0, 2, 1, 3), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("H,Hkv", [(1, 1), (4, 4), (4, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 37), (2, 9), (4, 33), (7, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_sdpa(H, Hkv, Nq, Nk, causal):
    B, d = 2, 8
    q, k, v = _rand((B, Nq, H, d), 11), _rand((B, Nk, Hkv, d), 12), _rand((B, Nk, Hkv, d), 13)
    ro, rl = _torch_decode(q, k, v, causal, 0.41)
    o, lse = attn_decode(q, k, v, causal, 0.41)
    assert np.abs(o - ro).max() <= 1e-12 * max(1.0, np.abs(ro).max())
    assert np.abs(lse - rl).max() <= 1e-12 * max(1.0, np.abs(rl).max())


@pytest.mark.parametrize("causal", [False, True])
def test_decode_with_nq_equal_nk_is_prefill(causal):
    q, k, v = _rand((2, 13, 6, 8), 21), _rand((2, 13, 2, 8), 22), _rand((2, 13, 2, 8), 23)
    o, lse = attn_decode(q, k, v, causal, 0.3)
    ro, rl = attn_fwd_gqa(q, k, v, causal, 0.3)
    assert np.abs(o - ro).max() <= 1e-12 and np.abs(lse - rl).max() <= 1e-12


@pytest.mark.parametrize("Nq", [1, 3, 8])
def test_decode_is_last_rows_of_causal_prefill(Nq):
    Nk = 29
    qf, k, v = _rand((1, Nk, 4, 8), 31), _rand((1, Nk, 2, 8), 32), _rand((1, Nk, 2, 8), 33)
    po, pl = attn_fwd_gqa(qf, k, v, True, 0.5)
    o, lse = attn_decode(qf[:, Nk - Nq:], k, v, True, 0.5)
    assert np.abs(o - po[:, Nk - Nq:]).max() <= 1e-12
    assert np.abs(lse - pl[:, :, Nk - Nq:]).max() <= 1e-12


def test_single_query_causal_equals_noncausal():
    q, k, v = _rand((2, 1, 4, 8), 41), _rand((2, 50, 4, 8), 42), _rand((2, 50, 4, 8), 43)
    a, b = attn_decode(q, k, v, True, 0.2), attn_decode(q, k, v, False, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


_SPLITS = {
    "one": [(0, 40)],
    "even": [(0, 10), (10, 20), (20, 30), (30, 40)],
    "ragged": [(0, 1), (1, 17), (17, 39), (39, 40)],
    "with_empty_range": [(0, 0), (0, 25), (25, 40)],
    "tail_masked_for_early_rows": [(0, 37), (37, 40)],
}


@pytest.mark.parametrize("name", sorted(_SPLITS))
@pytest.mark.parametrize("causal", [False, True])
def test_split_and_merge_is_exact(name, causal):
    Nq, Nk = 5, 40
    q, k, v = _rand((2, Nq, 4, 8), 51), _rand((2, Nk, 2, 8), 52), _rand((2, Nk, 2, 8), 53)
    ro, rl = attn_decode(q, k, v, causal, 0.35)
    o, lse = attn_decode_split(q, k, v, causal, 0.35, _SPLITS[name])
    assert np.abs(o - ro).max() <= 1e-12 and np.abs(lse - rl).max() <= 1e-12


def test_fully_masked_chunk_is_neutral():
    # Nq = 5 new tokens at positions 35..39: the chunk [37, 40) holds no visible key for rows 0 and 1.
    q, k, v = _rand((1, 5, 2, 8), 61), _rand((1, 40, 2, 8), 62), _rand((1, 40, 2, 8), 63)
    o, lse = attn_partial(q, k, v, True, 0.35, 37, 40)
    assert np.all(lse[0, :, :2] == -np.inf) and np.all(o[0, :2] == 0)
    assert np.all(np.isfinite(lse[0, :, 2:]))


def test_merge_identities():
    o1, l1 = attn_partial(*(_rand(s, i) for s, i in (((1, 3, 2, 4), 71), ((1, 9, 2, 4), 72), ((1, 9, 2, 4), 73))),
                          False, 0.5, 0, 4)
    o2, l2 = attn_partial(*(_rand(s, i) for s, i in (((1, 3, 2, 4), 71), ((1, 9, 2, 4), 72), ((1, 9, 2, 4), 73))),
                          False, 0.5, 4, 9)
    a = merge_partials([o1], [l1])
    assert np.allclose(a[0], o1, rtol=0, atol=1e-15) and np.allclose(a[1], l1, rtol=0, atol=1e-15)
    b, c = merge_partials([o1, o2], [l1, l2]), merge_partials([o2, o1], [l2, l1])
    assert np.abs(b[0] - c[0]).max() <= 1e-15 and np.abs(b[1] - c[1]).max() <= 1e-15
    # An empty partial (LSE = -inf) leaves the result unchanged.
    e = merge_partials([o1, np.zeros_like(o1)], [l1, np.full_like(l1, -np.inf)])
    assert np.allclose(e[0], o1, rtol=0, atol=1e-15) and np.allclose(e[1], l1, rtol=0, atol=1e-15)
    # LSE of the merge is the log-sum-exp of the partial LSEs (library routine).
    assert np.allclose(b[1], torch.logsumexp(torch.tensor(np.stack([l1, l2])), dim=0).numpy(), rtol=0, atol=1e-13)


def test_causal_needs_nq_at_most_nk():
    with pytest.raises(ValueError):
        attn_decode(_rand((1, 4, 1, 2), 1), _rand((1, 3, 1, 2), 2), _rand((1, 3, 1, 2), 3), True, 1.0)


def test_bytes_decode():
    # K and V of the cache dominate: 2 tensors x B*Nk*Hkv*d bf16 values.
    assert bytes_decode(1, 1, 1, 1, 1, 1) == 2 * 2 + 2 * 2 + 4
    assert bytes_decode(16, 32, 8, 1, 16384, 128) == 4.0 * 16 * 16384 * 8 * 128 + 4.0 * 16 * 32 * 128 + 4.0 * 16 * 32
