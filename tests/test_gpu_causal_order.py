"""Causal launches whose heads split evenly over the 8 XCDs start each XCD's blocks heaviest-first across
its heads (work_item in csrc/common.hpp): workgroup ids map to (head, block) differently from every other
launch. These cases use such head counts -- B*H (for grouped-query dK/dV: K/V heads times the split) a
multiple of 8 with at least two heads per XCD -- in every kernel form (forward with 4 and 8 waves at
d = 128 and 4 waves at d = 64, the paired and the 4-wave dK/dV kernels, dQ with 4 and 8 waves, the split
grouped-query dK/dV), and compare every output element with the fp64 oracle. Outputs start as NaN, so a
block that two workgroups computed while another was never computed would show.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import make_gqa, make_qkv
from oracle import attn_bwd, attn_fwd
from oracle.gqa import attn_bwd_gqa as ref_bwd_gqa
from oracle.gqa import attn_fwd_gqa as ref_fwd_gqa
from parity_util import DEV, TOL_GRAD_BF16, TOL_LSE_BF16, TOL_O_BF16, aerr, f64, nerr

pytestmark = pytest.mark.gpu


def _nan_like(t):
    return torch.full_like(t, float("nan"))


# (B, H, N, d): 16 heads; 700 tokens runs the 4-wave forward and dQ, 1500 the 8-wave forward and
# 4-wave dQ, 2200 both 8-wave; d = 64 runs the 4-wave dK/dV kernel.
CASES = [(2, 8, 700, 128), (2, 8, 1500, 128), (1, 16, 2200, 128), (2, 8, 700, 64)]


@pytest.mark.parametrize("B,H,N,d", CASES)
def test_causal_heaviest_first_order_covers_every_block(B, H, N, d):
    print(f"causal order: B={B} H={H} N={N} d={d}", flush=True)
    q, k, v, do = make_qkv(B, H, N, d, "bf16", seed=900 + N + d, with_do=True)
    s = float(np.float32(d ** -0.5))
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o = _nan_like(qd)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.attn_fwd(qd, kd, vd, True, s, o=o, lse=lse)
    dq, dk, dv = fa.attn_bwd(qd, kd, vd, o, dod, lse, True, s, dq=_nan_like(qd), dk=_nan_like(kd), dv=_nan_like(vd))
    torch.cuda.synchronize()
    qn, kn, vn, don = (x.double().numpy() for x in (q, k, v, do))
    ro, rl = attn_fwd(qn, kn, vn, True, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    rq, rk, rv = attn_bwd(qn, kn, vn, don, True, s)
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


def test_causal_heaviest_first_order_grouped_query():
    """16 query heads on 8 K/V heads: the forward's 16 units and the dK/dV grid over K/V heads and parts of
    their groups (split when the grouped-query workspace allows it)."""
    B, H, Hkv, N, d = 1, 16, 8, 700, 128
    q, k, v, do = make_gqa(B, H, Hkv, N, d, "bf16", seed=977, with_do=True)
    s = float(np.float32(d ** -0.5))
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o = _nan_like(qd)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.attn_fwd_gqa(qd, kd, vd, True, s, o=o, lse=lse)
    dq, dk, dv = fa.attn_bwd_gqa(qd, kd, vd, o, dod, lse, True, s, dq=_nan_like(qd), dk=_nan_like(kd),
                                 dv=_nan_like(vd))
    torch.cuda.synchronize()
    qn, kn, vn, don = (x.double().numpy() for x in (q, k, v, do))
    ro, rl = ref_fwd_gqa(qn, kn, vn, True, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    rq, rk, rv = ref_bwd_gqa(qn, kn, vn, don, True, s)
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16
