"""Run one stage of the attention path a few times, for profilers.

Usage: python -m exact_tiled_attention_13_amd.profile_run WHAT [--causal] [--reps R]
WHAT is one of fwd, bwd_prep, bwd_dq, bwd_dq_prep (dQ with the preprocess
fused, as attn_bwd runs it), bwd_dkdv, step (fwd, bwd_dq_prep, bwd_dkdv: one
forward and backward as bench.py times them), fp8, decode, fwd_short (the
forward of the short-sequence workload: batch 32, 32 heads, 512 tokens, head
dim 64), or copy (a plain device-to-device copy of 256 MiB through torch, used to
calibrate the HBM byte counters: it reads and writes exactly 256 MiB per
launch).
Workloads: batch 1, 16 heads, 16384 tokens, head dim 128, seeded inputs, bf16
(fwd .. step) or E4M3 (fp8); decode: 16 sequences, 32 query heads on 8 K/V
heads, one new token (four with --causal) against a 16384-token cache.
"""

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["fwd", "bwd_prep", "bwd_dq", "bwd_dq_prep", "bwd_dkdv", "step", "fp8",
                                        "decode", "fwd_short", "copy"])
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

    if args.what == "fp8":
        from exact_tiled_attention_13_amd.inputs import FP8_LONG, make_fp8

        w = FP8_LONG
        q8, k8, _, vt8, ds = make_fp8(w.B, w.H, w.N, w.d, w.seed)
        q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
        o, lse = fa.attn_fwd_fp8(q8, k8, vt8, *ds, args.causal, w.scale)
        for _ in range(args.reps):
            fa.attn_fwd_fp8(q8, k8, vt8, *ds, args.causal, w.scale, o=o, lse=lse)
        torch.cuda.synchronize()
        print(f"fp8 causal={args.causal} done", flush=True)
        return
    if args.what == "decode":
        from exact_tiled_attention_13_amd.inputs import DECODE_1, DECODE_4, make_decode

        w = DECODE_4 if args.causal else DECODE_1
        q, k, v = (x.to(dev) for x in make_decode(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed))
        o, lse = fa.attn_decode(q, k, v, args.causal, w.scale)
        ws = torch.empty(max(fa.attn_decode_workspace_size(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d), 256),
                         dtype=torch.uint8, device=dev)
        for _ in range(args.reps):
            fa.attn_decode(q, k, v, args.causal, w.scale, o=o, lse=lse, ws=ws)
        torch.cuda.synchronize()
        print(f"decode causal={args.causal} done", flush=True)
        return

    if args.what == "fwd_short":
        from exact_tiled_attention_13_amd.inputs import WORKLOADS

        w = WORKLOADS["fwd_bf16_b32_h32_n512_d64"]
        q, k, v = (x.to(dev) for x in make_workload(w))
        o, lse = fa.attn_fwd(q, k, v, args.causal, w.scale)
        for _ in range(args.reps):
            fa.attn_fwd(q, k, v, args.causal, w.scale, o=o, lse=lse)
        torch.cuda.synchronize()
        print(f"fwd_short causal={args.causal} done", flush=True)
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
        if args.what == "bwd_prep":
            fa.attn_bwd_prep(o, do, lse, ws=ws)
        if args.what == "bwd_dq":
            fa.attn_bwd_dq(q, k, v, do, ws, c, w.scale, dq=dq)
        if args.what in ("bwd_dq_prep", "step"):
            fa.attn_bwd_dq_prep(q, k, v, o, do, lse, ws=ws, causal=c, scale=w.scale, dq=dq)
        if args.what in ("bwd_dkdv", "step"):
            fa.attn_bwd_dkdv(q, k, v, do, ws, c, w.scale, dk=dk, dv=dv)
    torch.cuda.synchronize()
    print(f"{args.what} causal={c} done", flush=True)


if __name__ == "__main__":
    main()
