"""The backward's stages agree bitwise.

attn_bwd runs attn_bwd_dq_prep (dQ with the row statistics D_i and LSE_i * log2(e) formed in the dQ kernel)
and then attn_bwd_dkdv. attn_bwd_prep followed by attn_bwd_dq is the same first stage in two launches. The
fused kernel sums D_i in the same order as the separate preprocess, so both must leave the same workspace
(padded rows included) and the same dq, and attn_bwd must equal the three separate stages bit for bit. The
workspace starts filled with NaN bytes so that a row the fused kernel fails to write shows up.
"""

import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import make_qkv
from parity_util import DEV

pytestmark = pytest.mark.gpu

# (B, H, N, d): one-token and ragged sequences, the 4-wave dQ workgroup (d = 64, and d = 128 up to 2048
# tokens) and the 8-wave one (d = 128 beyond 2048 tokens).
SHAPES = [(1, 2, 1, 64), (2, 3, 100, 64), (1, 2, 1000, 128), (1, 2, 2113, 128), (1, 1, 4133, 64)]


def _stats(ws, B, H, N):
    npad = (N + 63) // 64 * 64
    return ws.view(torch.float32)[: 2 * B * H * npad]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_fused_preprocess_matches_separate_stages(B, H, N, d, causal):
    print(f"fused prep: B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    scale = -0.2 if N == 1000 else None       # one case with a negative scale (sign folded into Q)
    q, k, v, do = (x.to(DEV) for x in make_qkv(B, H, N, d, "bf16", seed=40 + N, with_do=True))
    o, lse = fa.attn_fwd(q, k, v, causal, scale)

    ws_a = fa.workspace(B, H, N, d, DEV).fill_(0xFF)
    ws_b = fa.workspace(B, H, N, d, DEV).fill_(0xFF)
    fa.attn_bwd_prep(o, do, lse, ws=ws_a)
    dq_a = fa.attn_bwd_dq(q, k, v, do, ws_a, causal, scale)
    dk_a, dv_a = fa.attn_bwd_dkdv(q, k, v, do, ws_a, causal, scale)
    dq_b, _ = fa.attn_bwd_dq_prep(q, k, v, o, do, lse, ws=ws_b, causal=causal, scale=scale)
    dq_c, dk_c, dv_c = fa.attn_bwd(q, k, v, o, do, lse, causal, scale)
    torch.cuda.synchronize()

    sa, sb = _stats(ws_a, B, H, N), _stats(ws_b, B, H, N)
    assert not torch.isnan(sa).any()
    assert torch.equal(sa, sb)
    assert torch.equal(dq_a, dq_b)
    for x, y in ((dq_a, dq_c), (dk_a, dk_c), (dv_a, dv_c)):
        assert torch.equal(x, y)
