"""Race check: the parity cases of every kernel against the LDS-poison build.

``libfa_mi355x_ldspoison.so`` is built from the same sources with
``-DFA_LDS_POISON=1``: each kernel fills its LDS with 0xFF bytes (NaN in fp32
and bf16) and waits at a barrier before anything else. A kernel that reads
LDS no load or store of its own wrote -- a buffer handed between waves one
barrier too early, a tile consumed before its loads landed, a lagging wave
reading a stage already refilled with uninitialised bytes -- then returns
NaN (nerr rejects non-finite values) or, if the poison happens to be
overwritten by stale data of a previous tile, values outside the tolerance.
Equality of results across the two builds is not required: the normal
build's LDS holds whatever the previous workgroup left, which is exactly what
this check removes.

The shapes cover every kernel and launch form: the forward at d = 64 and 128
with 4- and 8-wave workgroups, ragged and causal tails, the fp32 forward, the
backward (the dQ kernel with the row statistics formed in it, the 4-wave
d = 64 dK/dV kernel, the paired d = 128 kernel whose dS wave lags its P wave
by one tile; the separate preprocess through the stage tests of the suite
run against this build), the split grouped-
query dK/dV with its reduction, decoding and the FP8 forward.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import make_decode, make_fp8, make_qkv
from oracle import attn_bwd, attn_bwd_gqa, attn_fwd
from oracle.decode import attn_decode as ref_decode
from oracle.fp8 import attn_fwd_fp8 as ref_fp8
from parity_util import DEV, TOL_GRAD_BF16, TOL_LSE_BF16, TOL_LSE_FP32, TOL_O_BF16, TOL_O_FP32, aerr, f64, nerr

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def poison_library():
    with fa.use_library(fa.LIB_POISON_PATH):
        yield


@pytest.mark.parametrize("N,d", [(100, 64), (1000, 128), (2113, 128), (2113, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_poison_fwd_bwd(N, d, causal):
    print(f"poison fwd/bwd N={N} d={d} causal={causal}", flush=True)
    q, k, v, do = make_qkv(1, 2, N, d, "bf16", seed=900 + N + d + causal, with_do=True)
    s = float(np.float32(d ** -0.5))
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attn_fwd(qd, kd, vd, causal, s)
    dq, dk, dv = fa.attn_bwd(qd, kd, vd, o, dod, lse, causal, s)
    torch.cuda.synchronize()
    n = lambda t: t.double().numpy()
    ro, rl = attn_fwd(n(q), n(k), n(v), causal, s)
    rq, rk, rv = attn_bwd(n(q), n(k), n(v), n(do), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_poison_fwd_fp32(causal):
    q, k, v = make_qkv(1, 2, 257, 64, "fp32", seed=901 + causal)
    s = float(np.float32(0.125))
    o, lse = fa.attn_fwd_fp32(q.to(DEV), k.to(DEV), v.to(DEV), causal, s)
    torch.cuda.synchronize()
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_FP32
    assert aerr(f64(lse), rl) <= TOL_LSE_FP32


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_poison_gqa_split(d, causal):
    B, H, Hkv, N = 1, 8, 1, 1000
    g = torch.Generator().manual_seed(902 + d + causal)
    q, do = (torch.randn(B, N, H, d, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(B, N, Hkv, d, generator=g).to(torch.bfloat16) for _ in range(2))
    s = float(np.float32(d ** -0.5))
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    assert fa.attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, causal) > fa.attn_bwd_workspace_size(B, H, N, d, causal)
    o, lse = fa.attn_fwd_gqa(qd, kd, vd, causal, s)
    dq, dk, dv = fa.attn_bwd_gqa(qd, kd, vd, o, dod, lse, causal, s)
    torch.cuda.synchronize()
    n = lambda t: t.double().numpy()
    rq, rk, rv = attn_bwd_gqa(n(q), n(k), n(v), n(do), causal, s)
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("Nq,causal", [(1, False), (4, True)])
def test_poison_decode(Nq, causal):
    q, k, v = make_decode(2, 8, 2, Nq, 3001, 128, 903 + Nq)
    o, lse = fa.attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), causal, 128 ** -0.5)
    torch.cuda.synchronize()
    ro, rl = ref_decode(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, 128 ** -0.5)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_poison_fp8(causal):
    N = 300
    q8, k8, v8, vt8, ds = make_fp8(1, 2, N, 128, 904 + causal)
    s = 128 ** -0.5
    o, lse = fa.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), vt8.to(DEV), *ds, causal, s)
    torch.cuda.synchronize()
    f = lambda t: t.view(torch.float8_e4m3fn).double().numpy()
    ro, rl, bound = ref_fp8(f(q8), f(k8), f(v8), *ds, causal, s, flip_eta="fp32")
    got = f64(o)
    assert np.isfinite(got).all()
    assert (np.abs(got - ro) <= bound + 2.0 ** -8 * np.abs(ro) + 1e-5 * np.abs(ro).max()).all()
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
