"""Benchmark of exact tiled attention (forward + backward) on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
at the long-context shape (batch 1, 16 heads, 16384 tokens, head dim 128,
bf16): forward and backward without the causal mask, then forward and
backward with it. Counted FLOP per pass: forward 4*B*H*N^2*d, backward 2.5x
that, both halved under the causal mask; the value is the step's counted
FLOP divided by its wall time, in TFLOP/s.

Each kernel launch is bracketed by HIP events on the stream it runs on, so
the average duration of every kernel is measured inside the timed region;
the dominant one is reported against its roofline. The fp64 CPU oracle is
timed on a bounded sample of the same workload as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-report]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % bf16 MFMA peak, 16k tokens/batch, d=64/128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published


TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def measured_traffic(name: str):
    """HBM bytes per launch of kernel `name` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by the copy-kernel calibration), or
    None when no such measurement exists for the current kernel source."""
    try:
        with open(TRAFFIC) as f:
            entry = json.load(f)["kernels"].get(name)
    except (OSError, ValueError, KeyError):
        return None
    from exact_tiled_attention_13_amd.traffic import kernel_source_hash

    if not entry or entry.get("source_sha256") != kernel_source_hash(name):
        return None
    return float(entry["hbm_bytes"])


def counted_fwd(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def cpu_baseline(q, k, v, do, scale, heads=2, refs=None):
    """Time the fp64 oracle on a bounded sample of the step: the whole step
    (forward and backward, both masks) for the first `heads` heads. The oracle's
    outputs go into `refs[(causal, h)]` when a dict is given."""
    from threadpoolctl import threadpool_info

    from oracle import attn_bwd_head

    B, N, H, d = q.shape
    t0 = time.perf_counter()
    flops = 0.0
    for h in range(heads):
        qh, kh, vh, gh = (x[0, :, h].double().numpy() for x in (q, k, v, do))
        for causal in (False, True):
            # attn_bwd_head runs the oracle forward (O, LSE) and the backward.
            r = attn_bwd_head(qh, kh, vh, gh, causal, scale)
            if refs is not None:
                refs[(causal, h)] = r
            flops += 3.5 * counted_fwd(1, 1, N, d, causal)
    t1 = time.perf_counter()
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {
        "value": flops / (t1 - t0) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle running the whole step (forward and backward, non-causal and causal) "
                   f"for {heads} of the {H} heads of the same inputs, {t1 - t0:.1f} s; value uses the "
                   f"same counted-FLOP formula as the GPU step"),
        "seconds": round(t1 - t0, 2),
        "cpu_model": cpu,
        "blas": ", ".join(f"{i.get('internal_api', '?')} {i.get('version', '')} ({i.get('num_threads', 1)} threads)"
                          for i in blas) or "none found",
    }


def step_errors(bufs, refs):
    """Max normalised error (max |gpu - oracle| / max |oracle| over the checked elements) of the timed
    step's outputs O, dQ, dK, dV, and the max absolute LSE error, per mask, over the heads in `refs`
    (whole heads: every query and key row). Runs after the timed region."""
    import numpy as np

    out = {}
    for causal in (False, True):
        hs = sorted(h for (c, h) in refs if c == causal)
        if not hs:
            continue
        b = bufs[causal]
        got = {n: b[n][0].float().cpu().double().numpy() for n in ("o", "dq", "dk", "dv")}
        lse = b["lse"][0].cpu().double().numpy()
        e = {}
        for n in ("o", "dq", "dk", "dv"):
            g = np.concatenate([got[n][:, h] for h in hs])
            r = np.concatenate([refs[(causal, h)][n] for h in hs])
            e[n] = float(np.abs(g - r).max() / np.abs(r).max())
        e["lse_abs"] = float(max(np.abs(lse[h] - refs[(causal, h)]["lse"]).max() for h in hs))
        e["heads"] = hs
        out["causal" if causal else "noncausal"] = {k: (round(v, 6) if isinstance(v, float) else v)
                                                    for k, v in e.items()}
    out["tolerance"] = {"o": 2e-2, "dq_dk_dv": 5e-2, "lse_abs": 1e-3}
    return out


def _raw(name, *args):
    """A zero-argument call of the library's C entry point `name` with fixed arguments (device pointers as
    ints, sizes, the stream). Timing loops of the short report workloads use it so that the Python binding's
    per-call checks (tens of microseconds) do not pace kernels of about 0.1 ms; the same arguments went
    through the binding's checks once before."""
    import exact_tiled_attention_13_amd as fa

    fn = getattr(fa.lib(), name)
    return lambda: fn(*args)


def _time_calls(f, reps, warmup, min_warm_ms=20.0, min_timed_ms=50.0):
    """Mean ms of back-to-back calls of f (returning a library status) between two HIP events on the
    current stream. Short calls are repeated until the untimed warm-up covers at least min_warm_ms and the
    timed loop at least min_timed_ms of GPU time (and at least `warmup` / `reps` calls): a loop of ten
    0.1 ms calls straight after the host has been preparing inputs runs partly before the GPU's clocks have
    come back up and reads up to 20% slow."""
    import math

    import torch

    def run(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bad = 0
        e0.record()
        for _ in range(n):
            bad |= f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), bad

    t, bad = run(warmup)
    if bad:
        raise RuntimeError("library call failed during warmup")
    est = max(t / max(warmup, 1), 1e-3)
    t, bad = run(max(0, math.ceil(min_warm_ms / est) - warmup))
    if bad:
        raise RuntimeError("library call failed during warmup")
    n = max(reps, math.ceil(min_timed_ms / est))
    t, bad = run(n)
    if bad:
        raise RuntimeError("library call failed in the timed loop")
    return t / n


def time_passes(w, reps=10, warmup=3):
    """Report-only timing of one workload: forward (and backward, when the
    workload has one) for each of its masks, HIP events around `reps`
    back-to-back launches after `warmup` untimed ones."""
    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import make_workload

    dev = torch.device("cuda:0")
    xs = [x.to(dev) for x in make_workload(w)]
    q, k, v = xs[:3]
    out = {}
    gqa = w.kv_heads != w.H
    fwd = fa.attn_fwd_gqa if gqa else fa.attn_fwd
    bwd = fa.attn_bwd_gqa if gqa else fa.attn_bwd
    st = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr()
    heads = (w.B, w.H, w.kv_heads) if gqa else (w.B, w.H)
    for c in w.causal:
        tag = "causal" if c else "noncausal"
        o, lse = fwd(q, k, v, c, w.scale)
        calls = {"fwd": (_raw("attn_fwd_gqa" if gqa else "attn_fwd", p(q), p(k), p(v), p(o), p(lse), *heads,
                              w.N, w.d, int(c), w.scale, st), 1.0)}
        if w.backward:
            ws = (fa.workspace_gqa(w.B, w.H, w.kv_heads, w.N, w.d, c, dev) if gqa
                  else fa.workspace(w.B, w.H, w.N, w.d, dev))
            dq, dk, dv = bwd(q, k, v, o, xs[3], lse, c, w.scale, workspace=ws)
            calls["bwd"] = (_raw("attn_bwd_gqa" if gqa else "attn_bwd", p(q), p(k), p(v), p(o), p(xs[3]), p(lse),
                                 p(dq), p(dk), p(dv), p(ws), ws.numel(), *heads, w.N, w.d, int(c), w.scale, st),
                            2.5)
        for name, (f, mult) in calls.items():
            ms = _time_calls(f, reps, warmup)
            flop = mult * counted_fwd(w.B, w.H, w.N, w.d, c)
            out[f"{name}_{tag}"] = {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                                    "frac_bf16_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    return out


def time_sweep(reps=10, warmup=3):
    """Report-only: the pages' kernel benchmark grid (inputs.SWEEP_*): for each sequence length, head dim
    and mask, the forward and the backward at 16k tokens per batch, timed as time_passes times them."""
    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import SWEEP_D, SWEEP_N, make_qkv_device, sweep_shape

    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr()
    out = {}
    for d in SWEEP_D:
        for N in SWEEP_N:
            B, H, _, _ = sweep_shape(N, d)
            q, k, v, do = make_qkv_device(B, H, N, d, seed=2000 + N + d, device=dev)
            scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
            ws = fa.workspace(B, H, N, d, dev)
            for c in (False, True):
                o, lse = fa.attn_fwd(q, k, v, c, scale)
                dq, dk, dv = fa.attn_bwd(q, k, v, o, do, lse, c, scale, workspace=ws)
                fwd = _raw("attn_fwd", p(q), p(k), p(v), p(o), p(lse), B, H, N, d, int(c), scale, st)
                bwd = _raw("attn_bwd", p(q), p(k), p(v), p(o), p(do), p(lse), p(dq), p(dk), p(dv), p(ws),
                           ws.numel(), B, H, N, d, int(c), scale, st)
                entry = {"B": B, "H": H}
                for name, f, mult in (("fwd", fwd, 1.0), ("bwd", bwd, 2.5)):
                    ms = _time_calls(f, reps, warmup)
                    flop = mult * counted_fwd(B, H, N, d, c)
                    entry[f"{name}_ms"] = round(ms, 4)
                    entry[f"{name}_frac_bf16_peak"] = round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
                out[f"n{N}_d{d}_{'causal' if c else 'noncausal'}"] = entry
            del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def decode_bytes(B, H, Hkv, Nq, Nk, d):
    """Compulsory HBM bytes of one bf16 decode call: K and V of the cache, Q, O (bf16) and LSE (fp32)."""
    return 2.0 * 2 * B * Nk * Hkv * d + 2.0 * 2 * B * Nq * H * d + 4.0 * B * H * Nq


def time_decode(w, reps=20, warmup=5):
    """Report-only timing of a decoding workload (attn_decode: split kernel and merge), HIP events around
    `reps` back-to-back calls; the rate is compulsory bytes over time against the 8 TB/s HBM peak."""
    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import make_decode

    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in make_decode(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed))
    ws = torch.empty(fa.attn_decode_workspace_size(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d), dtype=torch.uint8, device=dev)
    out = {}
    st = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr()
    for c in w.causal:
        o, lse = fa.attn_decode(q, k, v, c, w.scale, ws=ws)
        f = _raw("attn_decode", p(q), p(k), p(v), p(o), p(lse), p(ws), ws.numel(), w.B, w.H, w.Hkv, w.Nq, w.Nk,
                 w.d, int(c), w.scale, st)
        ms = _time_calls(f, reps, warmup)
        gbs = decode_bytes(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d) / ms / 1e6
        out["decode_" + ("causal" if c else "noncausal")] = {
            "ms": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published


def time_fp8(w, reps=10, warmup=3):
    """Report-only timing of the FP8 (E4M3) forward at a workload's shape, both of its masks; counted FLOP
    as for the bf16 forward, against the fp8 and the bf16 dense peaks."""
    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import make_fp8

    dev = torch.device("cuda:0")
    q8, k8, _, vt8, ds = make_fp8(w.B, w.H, w.N, w.d, w.seed)
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    out = {}
    st = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr()
    for c in w.causal:
        o, lse = fa.attn_fwd_fp8(q8, k8, vt8, *ds, c, w.scale)
        f = _raw("attn_fwd_fp8", p(q8), p(k8), p(vt8), int(vt8.shape[3]), *ds, p(o), p(lse), w.B, w.H, w.N, w.d,
                 int(c), w.scale, st)
        ms = _time_calls(f, reps, warmup)
        tf = counted_fwd(w.B, w.H, w.N, w.d, c) / ms / 1e9
        out["fwd_fp8_" + ("causal" if c else "noncausal")] = {
            "ms": round(ms, 4), "tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-report", action="store_true", help="skip the report-only timings (the other workloads and the sweep)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(across GPUs the kernels would shard by heads, with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import BWD_LONG, make_workload

    w = BWD_LONG
    B, H, N, d = w.B, w.H, w.N, w.d
    dev = torch.device("cuda:0")
    q, k, v, do = make_workload(w)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    masks = (False, True)
    bufs = {}
    for c in masks:
        bufs[c] = dict(o=torch.empty_like(qd), lse=torch.empty((B, H, N), dtype=torch.float32, device=dev),
                       ws=fa.workspace(B, H, N, d, dev), dq=torch.empty_like(qd),
                       dk=torch.empty_like(kd), dv=torch.empty_like(vd))
    scale = w.scale
    stream = torch.cuda.current_stream(dev)

    names = []
    for c in masks:
        tag = "causal" if c else "noncausal"
        names += [f"fwd_{tag}", f"bwd_dq_prep_{tag}", f"bwd_dkdv_{tag}"]

    # The backward as attn_bwd runs it: dQ with the row statistics formed in
    # its kernel (attn_bwd_dq_prep), then dK/dV.
    def launches(c):
        b = bufs[c]
        return [
            lambda: fa.attn_fwd(qd, kd, vd, c, scale, o=b["o"], lse=b["lse"]),
            lambda: fa.attn_bwd_dq_prep(qd, kd, vd, b["o"], dod, b["lse"], ws=b["ws"], causal=c, scale=scale,
                                        dq=b["dq"]),
            lambda: fa.attn_bwd_dkdv(qd, kd, vd, dod, b["ws"], c, scale, dk=b["dk"], dv=b["dv"]),
        ]

    calls = [f for c in masks for f in launches(c)]

    def step(events=None):
        for i, f in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            f()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(args.steps)]
    from exact_tiled_attention_13_amd.gpuinfo import ClockSampler, device_facts

    torch.cuda.synchronize()
    with ClockSampler(dev) as clocks:
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(ev[s])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    launch_ms = {n: sorted(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps))
                 for i, n in enumerate(names)}
    kern_ms = {n: sum(v) / len(v) for n, v in launch_ms.items()}
    kern_med = {n: (v[(len(v) - 1) // 2] + v[len(v) // 2]) / 2 for n, v in launch_ms.items()}

    # Algorithmic work per launch.
    work = {}
    for c in masks:
        tag = "causal" if c else "noncausal"
        f1 = counted_fwd(B, H, N, d, c) / 2           # one N x N x d product
        work[f"fwd_{tag}"] = ("mfma", 2 * f1)
        work[f"bwd_dkdv_{tag}"] = ("mfma", 4 * f1)     # S (recompute), dP, dV, dK
        work[f"bwd_dq_prep_{tag}"] = ("mfma", 1 * f1)  # dQ (S, dP recomputed again: not counted)
    step_flops = sum(counted_fwd(B, H, N, d, c) * 3.5 for c in masks)

    breakdown = {}
    for n in names:
        kind, amount = work[n]
        rate = amount / (kern_ms[n] * 1e-3)
        if kind == "mfma":
            breakdown[n] = {"ms": round(kern_ms[n], 4), "tflops": round(rate / 1e12, 1),
                            "frac_bf16_peak": round(rate / 1e12 / PEAK_BF16_TFLOPS, 4)}
        else:
            breakdown[n] = {"ms": round(kern_ms[n], 4), "gbs": round(rate / 1e9, 1),
                            "frac_hbm_peak": round(rate / 1e9 / PEAK_HBM_GBS, 4)}
        # Mean (above), median and minimum over the timed steps' launches.
        breakdown[n]["ms_median"] = round(kern_med[n], 4)
        breakdown[n]["ms_min"] = round(launch_ms[n][0], 4)
    passes = {}
    for c in masks:
        tag = "causal" if c else "noncausal"
        fms = kern_ms[f"fwd_{tag}"]
        bms = kern_ms[f"bwd_dq_prep_{tag}"] + kern_ms[f"bwd_dkdv_{tag}"]
        ff = counted_fwd(B, H, N, d, c)
        passes[f"fwd_{tag}"] = {"ms": round(fms, 4), "tflops": round(ff / fms / 1e9, 1),
                                "frac_bf16_peak": round(ff / fms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        passes[f"bwd_{tag}"] = {"ms": round(bms, 4), "tflops": round(2.5 * ff / bms / 1e9, 1),
                                "frac_bf16_peak": round(2.5 * ff / bms / 1e9 / PEAK_BF16_TFLOPS, 4)}

    dom = max(names, key=lambda n: kern_ms[n])
    kind, amount = work[dom]
    achieved = amount / (kern_ms[dom] * 1e-3)
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / 1e9 / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom)}
    roof["kernel"] = dom
    roof["work_per_launch"] = amount
    roof["avg_launch_ms"] = round(kern_ms[dom], 4)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention forward+backward, non-causal then causal, B=1 H=16 N=16384 d=128 "
                               "(16k tokens per batch), bf16 in / fp32 accumulate",
                   "B": B, "H": H, "N": N, "d": d, "causal": list(masks), "seed": w.seed},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "passes": passes,
        "kernels": breakdown,
        "roofline": roof,
        "gpu": device_facts(dev),
        "clocks_timed_region": clocks.summary(),
        "max_memory_allocated_bytes": int(torch.cuda.max_memory_allocated(dev)),
    }
    # The matrix cores' sustained rate on this machine, measured after the timed region (reported beside the
    # published 2.5 PF denominator, never in its place): back-to-back MFMAs on every SIMD with constant
    # operands, and with changing pseudo-random operands, whose switching power lowers the clock.
    from exact_tiled_attention_13_amd import micro

    out["mfma_microbench"] = {f"operands_{name}": micro.mfma_bf16(dev, mode=m)
                              for name, m in (("constant", 0), ("random", 1))}
    # Each pass's rate as a share of that measured changing-operand rate: how much of what this box's
    # matrix cores sustain under the power limit the pass gets (context for box-to-box differences).
    mf = out["mfma_microbench"]["operands_random"]["tflops"]
    for p_ in passes.values():
        p_["frac_measured_mfma"] = round(p_["tflops"] / mf, 4) if mf > 0 else None
    # Report-only: the other 16k-token workloads (head dim 64 at 16k tokens,
    # grouped-query attention at 16k tokens, the short-sequence and mid-length
    # configurations, the batched backward), decoding against a 16k-token
    # cache (HBM-bound: reported in GB/s) and the FP8 forward at 16k tokens.
    from exact_tiled_attention_13_amd.inputs import LONG_D64, LONG_GQA, WORKLOADS

    if not args.no_report:
        report = {LONG_D64.name: time_passes(LONG_D64), LONG_GQA.name: time_passes(LONG_GQA)}
        for name in ("fwd_bf16_b32_h32_n512_d64", "fwd_bf16_b8_h16_n2048_d128", "bwd_bf16_b4_h16_n4096_d128"):
            report[name] = time_passes(WORKLOADS[name])
        from exact_tiled_attention_13_amd.inputs import DECODE_1, DECODE_4

        for dw in (DECODE_1, DECODE_4):
            report[dw.name] = time_decode(dw)
        from exact_tiled_attention_13_amd.inputs import FP8_LONG

        report[FP8_LONG.name] = time_fp8(FP8_LONG)
        out["other_workloads"] = report
        # The pages' sweep: sequence lengths 512 .. 16384 at 16k tokens per batch, d = 64 and 128, both masks.
        out["sweep_16k_tokens"] = time_sweep()
    refs = {}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, do, scale, refs=refs)
    else:
        # Parity of the timed outputs still checked, on one head per mask.
        from oracle import attn_bwd_head

        for c in masks:
            refs[(c, 0)] = attn_bwd_head(*(x[0, :, 0].double().numpy() for x in (q, k, v, do)), c, scale)
    out["parity_timed_step"] = step_errors(bufs, refs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
