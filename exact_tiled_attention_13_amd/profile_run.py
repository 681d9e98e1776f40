"""Run one stage of the attention path a few times, for profilers.

Usage: python -m exact_tiled_attention_13_amd.profile_run WHAT [--causal] [--reps R]
WHAT is one of fwd, bwd_prep, bwd_dkdv, bwd_dq, step (all four), or copy
(a plain device-to-device copy of 256 MiB through torch, used to calibrate
the HBM byte counters: it reads and writes exactly 256 MiB per launch).
Workload: batch 1, 16 heads, 16384 tokens, head dim 128, bf16, seeded inputs.
"""

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["fwd", "bwd_prep", "bwd_dkdv", "bwd_dq", "step", "copy"])
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()

    import torch

    import exact_tiled_attention_13_amd as fa
    from exact_tiled_attention_13_amd.inputs import BWD_LONG, make_workload

    dev = torch.device("cuda:0")
    if args.what == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy done", flush=True)
        return

    w = BWD_LONG
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v, do = (x.to(dev) for x in make_workload(w))
    c = args.causal
    o, lse = fa.attn_fwd(q, k, v, c, w.scale)
    ws = fa.attn_bwd_prep(o, do, lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        if args.what in ("fwd", "step"):
            fa.attn_fwd(q, k, v, c, w.scale, o=o, lse=lse)
        if args.what in ("bwd_prep", "step"):
            fa.attn_bwd_prep(o, do, lse, ws=ws)
        if args.what in ("bwd_dkdv", "step"):
            fa.attn_bwd_dkdv(q, k, v, do, ws, c, w.scale, dk=dk, dv=dv)
        if args.what in ("bwd_dq", "step"):
            fa.attn_bwd_dq(q, k, v, do, ws, c, w.scale, dq=dq)
    torch.cuda.synchronize()
    print(f"{args.what} causal={c} done", flush=True)


if __name__ == "__main__":
    main()
