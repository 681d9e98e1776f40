"""GPU parity of the FP8 (E4M3) forward (attn_fwd_fp8, through the C ABI)
against the FP8 oracle (oracle.fp8), which follows the same steps in fp64:
exact scores of the E4M3 inputs, the online softmax over 64-key tiles with
the exact running maximum, P rounded to E4M3 for the P V product and the row
sum from the unrounded P. Shapes span one to many tiles with ragged tails,
both masks, grouped batches and heads, and a negative scale.

Tolerance. The GPU rounds a P computed from scores summed on the FP8 matrix
cores, the oracle one computed in fp64; where P lies within that error of an
E4M3 rounding boundary the two pick neighbouring values, 2^-3 apart. So each
element of O must lie within the oracle's bound: the largest move of that
element if every P within eta of a boundary rounded the other way (eta from
the score error bound of oracle.fp8.fp32_p_error under the matrix cores'
accumulation model, which tests/test_gpu_fp8_mfma_accum.py measures on the
device), plus the error of the P V and row sums,
the bf16 rounding of the output (2^-8 relative) and 1e-5 of max|O|; LSE,
which uses the unrounded P, within 1e-3 as for bf16."""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import FP8_LONG, make_fp8
from oracle.fp8 import attn_fwd_fp8 as ref_fp8
from oracle.fp8 import attn_fwd_fp8_head
from parity_util import DEV, TOL_LSE_BF16, aerr, f64, sample_rows

pytestmark = pytest.mark.gpu


def run(q8, k8, vt8, ds, causal, scale):
    o, lse = fa.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), vt8.to(DEV), *ds, causal, scale)
    torch.cuda.synchronize()
    return o, lse


def check(B, H, N, causal, scale, seed, heads=None):
    print(f"fp8 B={B} H={H} N={N} causal={causal} scale={scale}", flush=True)
    q8, k8, v8, vt8, ds = make_fp8(B, H, N, 128, seed)
    o, lse = run(q8, k8, vt8, ds, causal, scale)
    hs = range(H) if heads is None else heads
    sel = lambda t: t.to(torch.float64).numpy()[:, :, list(hs)]
    ro, rl, bound = ref_fp8(sel(q8), sel(k8), sel(v8), *ds, causal, scale, flip_eta="fp32")
    got = f64(o)[:, :, list(hs)]
    assert np.isfinite(got).all()
    excess = np.abs(got - ro) - (bound + 2.0 ** -8 * np.abs(ro) + 1e-5 * np.abs(ro).max())
    assert excess.max() <= 0, (float(excess.max()), float(np.abs(got - ro).max()), float(bound.max()))
    # The envelope is not vacuous: on average it is under a tenth of what rounding every P to E4M3 may move
    # O by (2^-4 of sum_j P_j |v_j| / l, about 2^-4 of the mean |v|).
    assert bound.mean() <= 0.1 * 2.0 ** -4 * np.abs(sel(v8) * ds[2]).mean()
    assert aerr(f64(lse)[:, list(hs)], rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 2, 64), (2, 3, 100), (1, 2, 257), (2, 2, 1000), (1, 4, 2049)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_shapes(B, H, N, causal):
    check(B, H, N, causal, 128 ** -0.5, 3000 + B + 7 * H + N)


def test_fp8_negative_scale():
    check(2, 2, 333, True, -0.11, 3101)


def test_fp8_long_sampled_heads():
    # The long-context shape on two of its heads (the oracle runs them in full).
    w = FP8_LONG
    for causal in w.causal:
        check(w.B, w.H, 4096, causal, w.scale, w.seed, heads=[0, 9])


def test_fp8_timed_shape_sampled_rows():
    """The exact inputs the benchmark times (1 x 16 heads x 16384 tokens, seed of the FP8 workload), both
    masks, in the benchmark's launch configuration: sampled rows of three heads against the oracle, which
    computes each selected row over all 16384 keys in the same 64-key tiles."""
    w = FP8_LONG
    q8, k8, v8, vt8, ds = make_fp8(w.B, w.H, w.N, w.d, w.seed)
    for causal in w.causal:
        print(f"fp8 timed shape causal={causal}", flush=True)
        o, lse = run(q8, k8, vt8, ds, causal, w.scale)
        o, lse = o.cpu(), lse.cpu()
        for i, h in enumerate([0, 7, 15]):
            rows = sample_rows(w.N, 96, seed=w.seed + i)
            x = lambda t, s: t[0, :, h].to(torch.float64).numpy() * s
            ro, rl, bound = attn_fwd_fp8_head(x(q8, ds[0]), x(k8, ds[1]), x(v8, ds[2]), causal, w.scale,
                                              flip_eta="fp32", rows=rows)
            got = f64(o[0, rows, h])
            assert np.isfinite(got).all()
            excess = np.abs(got - ro) - (bound + 2.0 ** -8 * np.abs(ro) + 1e-5 * np.abs(ro).max())
            assert excess.max() <= 0, (causal, h, float(excess.max()))
            assert aerr(f64(lse[0, h, rows]), rl) <= TOL_LSE_BF16, (causal, h)


def test_fp8_pad_contents_do_not_matter():
    """Bytes N .. ldv-1 of each V^T row are padding: filled with 0x7F (an E4M3 NaN) instead of zeros, the
    output is bitwise unchanged (the kernel zeroes keys past N before the P V product)."""
    N = 1000                             # ragged: 1000 = 15 * 64 + 40
    q8, k8, v8, vt8, ds = make_fp8(1, 2, N, 128, 3301)
    for causal in (False, True):
        a = run(q8, k8, vt8, ds, causal, 0.09)
        bad = vt8.clone()
        bad[..., N:] = 0x7F
        b = run(q8, k8, bad, ds, causal, 0.09)
        assert torch.isfinite(b[0].float()).all()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_repeatable():
    q8, k8, v8, vt8, ds = make_fp8(1, 2, 700, 128, 3201)
    a = run(q8, k8, vt8, ds, True, 0.09)
    b = run(q8, k8, vt8, ds, True, 0.09)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
