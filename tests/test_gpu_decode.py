"""GPU parity of decoding (attn_decode, through the C ABI) against the fp64 CPU oracle.

Shapes cover one and several new tokens, multi-head, grouped-query and
multi-query heads up to the 32 query rows a K/V head can serve, caches that
are shorter than one 32-key tile, ragged, and long enough for hundreds of key
chunks, both masks, d = 64 and 128 and a negative scale. The decoding
workloads are compared on every row. A last test checks decoding against the
library's own prefill: the newest rows of a causal forward pass.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import DECODE_1, DECODE_4, make_decode
from oracle.decode import attn_decode as ref_decode
from parity_util import DEV, TOL_LSE_BF16, TOL_O_BF16, aerr, f64, nerr

pytestmark = pytest.mark.gpu


def run(q, k, v, causal, scale):
    o, lse = fa.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), causal, scale)
    torch.cuda.synchronize()
    return o, lse


def check(B, H, Hkv, Nq, Nk, d, causal, scale, seed):
    print(f"decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} scale={scale}", flush=True)
    q, k, v = make_decode(B, H, Hkv, Nq, Nk, d, seed)
    o, lse = run(q, k, v, causal, scale)
    ro, rl = ref_decode(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", [
    (1, 1, 1, 1, 1),          # one key
    (2, 4, 4, 1, 31),         # shorter than a tile
    (2, 4, 1, 1, 100),        # multi-query, ragged tail
    (3, 8, 2, 2, 257),        # groups of 4, two new tokens
    (1, 32, 1, 1, 1000),      # 32 query rows per K/V head
    (2, 8, 1, 4, 515),        # 32 rows: groups of 8, four tokens
    (1, 6, 3, 3, 64),         # exact tiles
    (1, 2, 2, 1, 5000),       # one K/V head per batch: ~150 key chunks
    (1, 4, 4, 7, 7),          # Nq = Nk: the whole sequence
])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_shapes(B, H, Hkv, Nq, Nk, causal, d):
    check(B, H, Hkv, Nq, Nk, d, causal, d ** -0.5, 2000 + B + 3 * H + 7 * Nq + Nk)


def test_decode_negative_scale():
    check(2, 8, 2, 3, 333, 128, True, -0.09, 2101)


@pytest.mark.parametrize("w", [DECODE_1, DECODE_4], ids=lambda w: w.name)
def test_decode_workloads(w):
    for causal in w.causal:
        check(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, causal, w.scale, w.seed)


def test_decode_matches_prefill_last_rows():
    # The newest Nq tokens decoded against the cache give the same rows as the
    # causal forward pass over the whole sequence (both on the GPU; the two
    # paths round differently, so within the forward tolerance).
    B, H, Hkv, N, d, Nq = 2, 8, 2, 700, 128, 5
    g = torch.Generator().manual_seed(2201)
    q = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, N, Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, N, Hkv, d, generator=g).to(torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    po, pl = fa.attn_fwd_gqa(qd, kd, vd, True, d ** -0.5)
    o, lse = fa.attn_decode(qd[:, N - Nq:].contiguous(), kd, vd, True, d ** -0.5)
    torch.cuda.synchronize()
    assert nerr(f64(o), f64(po[:, N - Nq:])) <= TOL_O_BF16
    assert aerr(f64(lse), f64(pl[:, :, N - Nq:])) <= TOL_LSE_BF16


def test_decode_is_deterministic_and_fills_outputs():
    q, k, v = make_decode(2, 8, 2, 2, 3000, 128, 2301)
    o1, l1 = run(q, k, v, True, 0.088)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    fa.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), True, 0.088, o=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.isfinite(f64(o2)).all() and np.isfinite(f64(l2)).all()
