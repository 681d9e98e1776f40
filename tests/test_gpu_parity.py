"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every case draws seeded inputs once on the CPU (exact_tiled_attention_13_amd.inputs),
runs the library on cuda:0 and the oracle on the identical values, and
compares with the tolerances in parity_util. Small and medium shapes are
compared element by element over whole tensors, with sizes that span several
tiles and a ragged tail; the full-size workloads are compared on sampled
heads and rows the oracle can compute one by one, in the same launch
configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as fa
from exact_tiled_attention_13_amd.inputs import BWD_LONG, WORKLOADS, make_qkv, make_workload
from oracle import attn_bwd_head, attn_fwd, attn_fwd_rows, attn_bwd
from parity_util import (DEV, TOL_GRAD_BF16, TOL_LSE_BF16, TOL_LSE_FP32, TOL_O_BF16, TOL_O_FP32, aerr, f64,
                         nerr, sample_rows)

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, causal, scale, fp32=False):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = (fa.attn_fwd_fp32 if fp32 else fa.attn_fwd)(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------------------
# fp32 forward

def test_fwd_fp32_workload():
    w = WORKLOADS["fwd_fp32_b1_h2_n128_d64"]
    q, k, v = make_workload(w)
    o, lse = run_fwd(q, k, v, False, w.scale, fp32=True)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), False, w.scale)
    assert nerr(f64(o), ro) <= TOL_O_FP32
    assert aerr(f64(lse), rl) <= TOL_LSE_FP32


@pytest.mark.parametrize("N", [1, 17, 100, 257, 600])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp32_shapes(N, d, causal):
    q, k, v = make_qkv(2, 3, N, d, "fp32", seed=N * 10 + d + causal)
    s = float(np.float32(d ** -0.5))
    o, lse = run_fwd(q, k, v, causal, s, fp32=True)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_FP32
    assert aerr(f64(lse), rl) <= TOL_LSE_FP32


# ---------------------------------------------------------------------------
# bf16 forward, whole-tensor comparison

@pytest.mark.parametrize("N", [1, 17, 100, 129, 257, 1000, 1024, 1025, 1537])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_shapes(N, d, causal):
    """Whole tensors against the oracle. At d = 128, 1025 tokens and more run
    the 8-wave ping-pong forward, 1024 and fewer the 4-wave one."""
    q, k, v = make_qkv(2, 3, N, d, "bf16", seed=N * 10 + d + causal + 7)
    s = float(np.float32(d ** -0.5))
    o, lse = run_fwd(q, k, v, causal, s)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_rising_scores(causal):
    """Scores that rise by about 16 (base 2) from each 64-key tile to the next: the 8-wave forward
    (1100 tokens at d = 128) takes every tile's exponentials against a running maximum that the tile
    then exceeds, so every tile goes through its rescale path (scores formed again, maximum moved, l
    and O rescaled)."""
    N, d = 1100, 128
    g = torch.Generator().manual_seed(5101 + causal)
    q = (0.1 + 0.02 * torch.randn(1, N, 2, d, generator=g)).to(torch.bfloat16)
    ramp = (10.0 * (torch.arange(N) // 64)).view(1, N, 1, 1)
    k = (ramp + torch.randn(1, N, 2, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, N, 2, d, generator=g).to(torch.bfloat16)
    s = float(np.float32(d ** -0.5))
    o, lse = run_fwd(q, k, v, causal, s)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16


def _sampled_rows_check(q, k, v, causal, scale, heads, nrows, seed):
    o, lse = (t.cpu() for t in run_fwd(q, k, v, causal, scale))
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for i, (b, h) in enumerate(heads):
        rows = sample_rows(q.shape[1], nrows, seed=seed + i)
        ro, rl = attn_fwd_rows(q[b, :, h].double().numpy(), k[b, :, h].double().numpy(),
                               v[b, :, h].double().numpy(), rows, causal, scale)
        got_o.append(f64(o[b, rows, h]))
        ref_o.append(ro)
        got_l.append(f64(lse[b, h, rows]))
        ref_l.append(rl)
    assert nerr(np.concatenate(got_o), np.concatenate(ref_o)) <= TOL_O_BF16
    assert aerr(np.concatenate(got_l), np.concatenate(ref_l)) <= TOL_LSE_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_long_d64_eight_wave(causal):
    """Head dim 64 from 4096 tokens on, on a grid of at least 512 eight-wave workgroups, runs the
    8-wave ping-pong forward (shorter sequences and smaller grids the 4-wave one): 2 x 16 heads x
    4097 tokens (17 query blocks of 256 per head, the last one row long) on sampled rows of three
    heads, the last row included."""
    N, d = 4097, 64
    q, k, v = make_qkv(2, 16, N, d, "bf16", seed=4097 + causal)
    s = float(np.float32(d ** -0.5))
    print(f"d64 eight-wave forward causal={causal}", flush=True)
    _sampled_rows_check(q, k, v, causal, s, heads=[(0, 0), (1, 7), (1, 15)], nrows=256, seed=77)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_rising_scores_d64(causal):
    """The rescale path of the 8-wave forward at d = 64 (1 x 32 heads x 4096 tokens, 512 eight-wave
    workgroups): scores rise by about 16 (base 2) from each 64-key tile to the next, so every tile
    outgrows the running maximum; sampled rows of three heads."""
    N, d, H = 4096, 64, 32
    g = torch.Generator().manual_seed(6101 + causal)
    q = (0.1 + 0.02 * torch.randn(1, N, H, d, generator=g)).to(torch.bfloat16)
    ramp = (14.0 * (torch.arange(N) // 64)).view(1, N, 1, 1)
    k = (ramp + torch.randn(1, N, H, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, N, H, d, generator=g).to(torch.bfloat16)
    s = float(np.float32(d ** -0.5))
    _sampled_rows_check(q, k, v, causal, s, heads=[(0, 0), (0, 13), (0, 31)], nrows=192, seed=91)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_other_scales(scale, causal):
    q, k, v = make_qkv(1, 2, 300, 64, "bf16", seed=55)
    o, lse = run_fwd(q, k, v, causal, scale)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16


def test_fwd_bf16_workload_n512_d64():
    """32 batches x 32 heads x 512 tokens, d 64, both masks: whole tensors."""
    w = WORKLOADS["fwd_bf16_b32_h32_n512_d64"]
    q, k, v = make_workload(w)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    for causal in w.causal:
        o, lse = run_fwd(q, k, v, causal, w.scale)
        ro, rl = attn_fwd(qn, kn, vn, causal, w.scale)
        assert nerr(f64(o), ro) <= TOL_O_BF16, causal
        assert aerr(f64(lse), rl) <= TOL_LSE_BF16, causal


def sampled_fwd_check(w, heads, nrows):
    q, k, v = make_workload(w)
    for causal in w.causal:
        o, lse = run_fwd(q, k, v, causal, w.scale)
        o, lse = o.cpu(), lse.cpu()
        got_o, ref_o, got_l, ref_l = [], [], [], []
        for i, (b, h) in enumerate(heads):
            rows = sample_rows(w.N, nrows, seed=w.seed + i)
            ro, rl = attn_fwd_rows(q[b, :, h].double().numpy(), k[b, :, h].double().numpy(),
                                   v[b, :, h].double().numpy(), rows, causal, w.scale)
            got_o.append(f64(o[b, rows, h]))
            ref_o.append(ro)
            got_l.append(f64(lse[b, h, rows]))
            ref_l.append(rl)
        assert nerr(np.concatenate(got_o), np.concatenate(ref_o)) <= TOL_O_BF16, causal
        assert aerr(np.concatenate(got_l), np.concatenate(ref_l)) <= TOL_LSE_BF16, causal


def test_fwd_bf16_workload_n2048_d128_sampled():
    w = WORKLOADS["fwd_bf16_b8_h16_n2048_d128"]
    sampled_fwd_check(w, heads=[(0, 0), (3, 7), (7, 15)], nrows=256)


def test_fwd_bf16_workload_n16384_d128_sampled():
    w = WORKLOADS["fwd_bf16_b1_h16_n16384_d128"]
    sampled_fwd_check(w, heads=[(0, 0), (0, 9), (0, 15)], nrows=192)


# ---------------------------------------------------------------------------
# bf16 backward

def run_bwd(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attn_fwd(qd, kd, vd, causal, scale)
    dq, dk, dv = fa.attn_bwd(qd, kd, vd, o, dod, lse, causal, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("N", [1, 17, 100, 257, 640])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_bf16_shapes(N, d, causal):
    q, k, v, do = make_qkv(2, 2, N, d, "bf16", seed=N * 3 + d + causal, with_do=True)
    s = float(np.float32(d ** -0.5))
    _, _, dq, dk, dv = run_bwd(q, k, v, do, causal, s)
    rq, rk, rv = attn_bwd(*(x.double().numpy() for x in (q, k, v, do)), causal, s)
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("scale", [-0.15, 0.0])
def test_bwd_bf16_other_scales(scale):
    q, k, v, do = make_qkv(1, 2, 200, 128, "bf16", seed=66, with_do=True)
    for causal in (False, True):
        _, _, dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
        rq, rk, rv = attn_bwd(*(x.double().numpy() for x in (q, k, v, do)), causal, scale)
        assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
        assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
        assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bwd_bf16_ragged_long_d128(causal):
    """Head dim 128 beyond 2048 tokens runs the 8-wave forward and dQ
    kernels (shorter sequences and d = 64 run the 4-wave ones); a ragged
    length (2113 = 33 * 64 + 1) checks their tail handling."""
    N = 2113
    q, k, v, do = make_qkv(1, 2, N, 128, "bf16", seed=2113 + causal, with_do=True)
    s = float(np.float32(128 ** -0.5))
    o, lse, dq, dk, dv = run_bwd(q, k, v, do, causal, s)
    ro, rl = attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    rq, rk, rv = attn_bwd(*(x.double().numpy() for x in (q, k, v, do)), causal, s)
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


def test_bwd_bf16_workload_n4096_sampled_heads():
    """4 x 16 heads x 4096 tokens, d 128, causal: O and LSE from the forward
    kernel feed the backward; three whole heads are checked against the oracle."""
    w = WORKLOADS["bwd_bf16_b4_h16_n4096_d128"]
    q, k, v, do = make_workload(w)
    causal = True
    o, lse, dq, dk, dv = (t.cpu() for t in run_bwd(q, k, v, do, causal, w.scale))
    got = {"o": [], "dq": [], "dk": [], "dv": []}
    ref = {"o": [], "dq": [], "dk": [], "dv": []}
    for b, h in [(0, 0), (2, 5), (3, 15)]:
        g = attn_bwd_head(*(x[b, :, h].double().numpy() for x in (q, k, v, do)), causal, w.scale)
        for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            got[name].append(f64(t[b, :, h]))
            ref[name].append(g[name])
        assert aerr(f64(lse[b, h]), g["lse"]) <= TOL_LSE_BF16
    assert nerr(np.concatenate(got["o"]), np.concatenate(ref["o"])) <= TOL_O_BF16
    for name in ("dq", "dk", "dv"):
        assert nerr(np.concatenate(got[name]), np.concatenate(ref[name])) <= TOL_GRAD_BF16, name


@pytest.mark.parametrize("causal,h", [(False, 3), (True, 12)])
def test_bwd_bf16_workload_n16384_d128_head(causal, h):
    """The timed long-context step (1 x 16 heads x 16384 tokens, d 128), in the
    launch configuration the benchmark times: the forward kernel's O and LSE
    feed the backward over all 16 heads; one whole head is checked against the
    oracle (every query row and every key row of that head)."""
    w = BWD_LONG
    q, k, v, do = make_workload(w)
    print(f"16k backward causal={causal} head={h}", flush=True)
    o, lse, dq, dk, dv = (t.cpu() for t in run_bwd(q, k, v, do, causal, w.scale))
    g = attn_bwd_head(*(x[0, :, h].double().numpy() for x in (q, k, v, do)), causal, w.scale)
    assert aerr(f64(lse[0, h]), g["lse"]) <= TOL_LSE_BF16
    assert nerr(f64(o[0, :, h]), g["o"]) <= TOL_O_BF16
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert nerr(f64(t[0, :, h]), g[name]) <= TOL_GRAD_BF16, name


# ---------------------------------------------------------------------------
# grouped-query / multi-query attention (K/V heads shared by query heads)

def run_gqa(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attn_fwd_gqa(qd, kd, vd, causal, scale)
    dq, dk, dv = fa.attn_bwd_gqa(qd, kd, vd, o, dod, lse, causal, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("H,Hkv", [(8, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("N", [17, 257])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bf16_shapes(H, Hkv, N, d, causal):
    from oracle import attn_bwd_gqa, attn_fwd_gqa
    g = torch.Generator().manual_seed(H * 100 + Hkv * 10 + N + d + causal)
    q, do = (torch.randn(2, N, H, d, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(2, N, Hkv, d, generator=g).to(torch.bfloat16) for _ in range(2))
    s = float(np.float32(d ** -0.5))
    o, lse, dq, dk, dv = run_gqa(q, k, v, do, causal, s)
    n = lambda t: t.double().numpy()
    ro, rl = attn_fwd_gqa(n(q), n(k), n(v), causal, s)
    rq, rk, rv = attn_bwd_gqa(n(q), n(k), n(v), n(do), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bf16_ragged_long_d128(causal):
    """8-wave forward and dQ kernels (d = 128 beyond 2048 tokens), two K/V heads for four query heads."""
    from oracle import attn_bwd_gqa, attn_fwd_gqa
    N = 2113
    g = torch.Generator().manual_seed(4242 + causal)
    q, do = (torch.randn(1, N, 4, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(1, N, 2, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    s = float(np.float32(128 ** -0.5))
    o, lse, dq, dk, dv = run_gqa(q, k, v, do, causal, s)
    n = lambda t: t.double().numpy()
    ro, rl = attn_fwd_gqa(n(q), n(k), n(v), causal, s)
    rq, rk, rv = attn_bwd_gqa(n(q), n(k), n(v), n(do), causal, s)
    assert nerr(f64(o), ro) <= TOL_O_BF16
    assert aerr(f64(lse), rl) <= TOL_LSE_BF16
    assert nerr(f64(dq), rq) <= TOL_GRAD_BF16
    assert nerr(f64(dk), rk) <= TOL_GRAD_BF16
    assert nerr(f64(dv), rv) <= TOL_GRAD_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bf16_long_d64_eight_wave_forward(causal):
    """The 8-wave d = 64 forward with grouped-query heads: 32 query heads on 4 K/V heads, 4096 tokens
    (512 eight-wave workgroups); sampled rows of query heads in three groups against the oracle on
    their K/V head."""
    from exact_tiled_attention_13_amd.inputs import make_gqa
    B, H, Hkv, N, d = 1, 32, 4, 4096, 64
    q, k, v = make_gqa(B, H, Hkv, N, d, "bf16", seed=4096 + causal)
    s = float(np.float32(d ** -0.5))
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.attn_fwd_gqa(qd, kd, vd, causal, s)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    G = H // Hkv
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for i, h in enumerate([0, 13, 31]):
        rows = sample_rows(N, 192, seed=300 + i)
        ro, rl = attn_fwd_rows(q[0, :, h].double().numpy(), k[0, :, h // G].double().numpy(),
                               v[0, :, h // G].double().numpy(), rows, causal, s)
        got_o.append(f64(o[0, rows, h]))
        ref_o.append(ro)
        got_l.append(f64(lse[0, h, rows]))
        ref_l.append(rl)
    assert nerr(np.concatenate(got_o), np.concatenate(ref_o)) <= TOL_O_BF16
    assert aerr(np.concatenate(got_l), np.concatenate(ref_l)) <= TOL_LSE_BF16


def test_gqa_with_hkv_equal_h_is_bitwise_mha():
    q, k, v, do = make_qkv(1, 3, 300, 64, "bf16", seed=77, with_do=True)
    s = float(np.float32(0.125))
    a = run_gqa(q, k, v, do, True, s)
    b = run_bwd(q, k, v, do, True, s)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gqa_bf16_workload_n16384_sampled():
    """The grouped-query workload the benchmark reports (16 query heads on 2 K/V
    heads, 16k tokens, d 128), in the same launch configuration: sampled rows of
    query heads in both groups against the oracle on their shared K/V head."""
    from exact_tiled_attention_13_amd.inputs import LONG_GQA as w
    q, k, v, _ = make_workload(w)
    G = w.H // w.kv_heads
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in w.causal:
        o, lse = fa.attn_fwd_gqa(qd, kd, vd, causal, w.scale)
        torch.cuda.synchronize()
        o, lse = o.cpu(), lse.cpu()
        got_o, ref_o, got_l, ref_l = [], [], [], []
        for i, h in enumerate([0, 7, 8, 15]):
            rows = sample_rows(w.N, 128, seed=w.seed + i)
            ro, rl = attn_fwd_rows(q[0, :, h].double().numpy(), k[0, :, h // G].double().numpy(),
                                   v[0, :, h // G].double().numpy(), rows, causal, w.scale)
            got_o.append(f64(o[0, rows, h]))
            ref_o.append(ro)
            got_l.append(f64(lse[0, h, rows]))
            ref_l.append(rl)
        assert nerr(np.concatenate(got_o), np.concatenate(ref_o)) <= TOL_O_BF16, causal
        assert aerr(np.concatenate(got_l), np.concatenate(ref_l)) <= TOL_LSE_BF16, causal
