"""Sequence-length sweep of the forward and backward passes, for reports.

Usage: python -m exact_tiled_attention_13_amd.sweep [--reps R] [--json FILE]

The grid is the kernel benchmark that the page "FlashAttention-2: atención
eficiente en GPU para contextos largos" describes in section "Qué significa
la mejora de aproximadamente dos veces": sequence lengths 512 to 16k at 16k
tokens per batch (B = 16384 / N), head dims 64 and 128 with H * d = 2048,
with and without the causal mask, forward and backward. Inputs are iid
N(0, 1) drawn on the GPU from a fixed seed and rounded to bf16 (timing only;
parity at these shapes is the tests' job). Each pass is timed with HIP events
around R back-to-back calls of the library's C entry points (forward:
attn_fwd; backward: attn_bwd, i.e. preprocess + dK/dV + dQ, from the
forward's O and LSE), repeated until the timed loop covers at least 50 ms
after at least 20 ms of untimed calls. Counted FLOP as everywhere
else: forward 4*B*H*N^2*d, backward 2.5x that, both halved under the causal
mask. Prints one JSON object per point and a markdown table.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
TOKENS = 16384
SEQ = (512, 1024, 2048, 4096, 8192, 16384)
HEADS = ((32, 64), (16, 128))


def _time(f, reps: int, min_warm_ms: float = 20.0, min_timed_ms: float = 50.0) -> float:
    """Mean ms per call over at least `reps` calls and min_timed_ms of GPU time,
    after at least min_warm_ms of untimed calls (so the clocks are up)."""
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
        if bad:
            raise RuntimeError("library call failed")
        return e0.elapsed_time(e1)

    est = max(run(2) / 2, 1e-3)
    run(max(0, math.ceil(min_warm_ms / est) - 2))
    n = max(reps, math.ceil(min_timed_ms / est))
    return run(n) / n


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--json", default=None, help="also write the points to this file")
    args = ap.parse_args()

    import torch

    import exact_tiled_attention_13_amd as fa

    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev).cuda_stream
    L = fa.lib()
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    P = lambda t: t.data_ptr()
    points = []
    for H, d in HEADS:
        for N in SEQ:
            B = TOKENS // N
            q, k, v, do = (torch.randn(B, N, H, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(4))
            o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
            lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
            ws = fa.workspace(B, H, N, d, dev)
            scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
            for causal in (False, True):
                c = int(causal)
                fa.attn_fwd(q, k, v, causal, scale, o=o, lse=lse)
                fwd = lambda: L.attn_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, c, scale, st)
                bwd = lambda: L.attn_bwd(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), P(ws),
                                         ws.numel(), B, H, N, d, c, scale, st)
                tf, tb = _time(fwd, args.reps), _time(bwd, args.reps)
                flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
                pt = {"B": B, "H": H, "N": N, "d": d, "causal": causal,
                      "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
                      "fwd_tflops": round(flop / tf / 1e9, 1), "bwd_tflops": round(2.5 * flop / tb / 1e9, 1),
                      "fwd_bwd_tflops": round(3.5 * flop / (tf + tb) / 1e9, 1)}
                for kk in ("fwd", "bwd", "fwd_bwd"):
                    pt[f"{kk}_frac_bf16_peak"] = round(pt[f"{kk}_tflops"] / PEAK_BF16_TFLOPS, 4)
                points.append(pt)
                print(json.dumps(pt), flush=True)
            del q, k, v, do, o, dq, dk, dv, lse, ws
            torch.cuda.empty_cache()
    if args.json:
        with open(args.json, "w") as fh:
            json.dump(points, fh, indent=1)
    print("\n| d | mask | pass | " + " | ".join(f"{n // 1024}k" if n >= 1024 else str(n) for n in SEQ) + " |")
    print("|---|---|---|" + "---|" * len(SEQ))
    for H, d in HEADS:
        for causal in (False, True):
            for kk in ("fwd", "bwd", "fwd_bwd"):
                row = [p for p in points if p["d"] == d and p["causal"] == causal]
                cells = " | ".join(f"{p[kk + '_tflops']:.0f} ({100 * p[kk + '_frac_bf16_peak']:.0f}%)" for p in row)
                print(f"| {d} | {'causal' if causal else 'none'} | {kk.replace('_', '+')} | {cells} |")


if __name__ == "__main__":
    main()
