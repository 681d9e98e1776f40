"""HBM bytes per kernel launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs.

Usage: python -m exact_tiled_attention_13_amd.traffic PROF_DIR [--out profiles/hbm_traffic.json]

PROF_DIR holds one rocprofv3 ``--pmc`` run per stage and counter, in
directories ``pmc_<stage>_<COUNTER>`` (stage: copy, fwd, bwd_dq_prep,
bwd_dkdv -- the kernels bench.py times; counter: FETCH_SIZE, WRITE_SIZE), each
made by

    rocprofv3 --pmc <COUNTER> --output-format csv -d PROF_DIR/pmc_<stage>_<COUNTER> -o run -- \\
        python3 -m exact_tiled_attention_13_amd.profile_run <stage> --reps 3

The ``copy`` stage copies 256 MiB per launch through the runtime's own copy
kernel: it reads and writes exactly 262144 KiB, so the ratio of that to what
each counter reports for it calibrates the counter. Every other stage's
counter is averaged over its launches of the stage's kernel (the backward
stages also launch the forward once, which is excluded), scaled, and stored
with the sha256 of the sources the kernel is built from; bench.py reports a
kernel's bytes only while that hash still matches.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
COPY_KIB = 262144

# Stage -> (kernel name prefix in the trace, name used by bench.py).
STAGES = {
    "fwd": ("fa::fwd_bf16_kernel<128, false, 8>", "fwd_noncausal"),
    "bwd_dq_prep": ("fa::bwd_dq_kernel<128, false, 8, true>", "bwd_dq_prep_noncausal"),
    "bwd_dkdv": ("fa::bwd_dkdv_pair_kernel<128, false, false>", "bwd_dkdv_noncausal"),
}


def kernel_source_hash(name: str) -> str:
    """sha256 over the sources and build script that kernel `name` (a bench.py
    kernel name such as ``bwd_dkdv_noncausal``) is compiled from."""
    main = "fwd_bf16.hip" if name.startswith("fwd") else "bwd_bf16.hip"
    h = hashlib.sha256()
    for f in [os.path.join(CSRC, x) for x in ("common.hpp", "lds_tile.hpp", "kernels.hpp", main)] + [
            os.path.join(PKG, "build.py")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _counter_kib(prof_dir: str, stage: str, counter: str, kernel: str | None) -> float:
    """Mean value of `counter` per launch of `kernel` (None: every launch)."""
    files = glob.glob(os.path.join(prof_dir, f"pmc_{stage}_{counter}", "**", "*counter_collection.csv"),
                      recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter collection for {stage} {counter} under {prof_dir}")
    per = {}
    for fn in files:
        with open(fn) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                if kernel is not None and kernel not in r["Kernel_Name"]:
                    continue
                key = (fn, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for {kernel} in {stage}")
    return sum(per.values()) / len(per)


def summarise(prof_dir: str) -> dict:
    fetch_scale = COPY_KIB / _counter_kib(prof_dir, "copy", "FETCH_SIZE", "copyBuffer")
    write_scale = COPY_KIB / _counter_kib(prof_dir, "copy", "WRITE_SIZE", "copyBuffer")
    out = {"calibration": {"copy_kib": COPY_KIB, "fetch_scale": fetch_scale, "write_scale": write_scale},
           "kernels": {}}
    for stage, (kernel, name) in STAGES.items():
        f = _counter_kib(prof_dir, stage, "FETCH_SIZE", kernel)
        w = _counter_kib(prof_dir, stage, "WRITE_SIZE", kernel)
        out["kernels"][name] = {"kernel": kernel.split("::")[1], "fetch_kib": f, "write_kib": w,
                                "hbm_bytes": 1024.0 * (f * fetch_scale + w * write_scale),
                                "source_sha256": kernel_source_hash(name)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("prof_dir")
    ap.add_argument("--out", default=os.path.join(os.path.dirname(PKG), "profiles", "hbm_traffic.json"))
    args = ap.parse_args()
    s = summarise(args.prof_dir)
    with open(args.out, "w") as fh:
        json.dump(s, fh, indent=1)
        fh.write("\n")
    print(f"calibration: FETCH_SIZE x {s['calibration']['fetch_scale']:.4f}, "
          f"WRITE_SIZE x {s['calibration']['write_scale']:.4f}")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MiB (scaled) | HBM write MiB |")
    print("|---|---|---|---|---|")
    for e in s["kernels"].values():
        print(f"| `{e['kernel']}` | {e['fetch_kib']:.0f} | {e['write_kib']:.0f} | "
              f"{e['fetch_kib'] * s['calibration']['fetch_scale'] / 1024:.1f} | "
              f"{e['write_kib'] * s['calibration']['write_scale'] / 1024:.1f} |")


if __name__ == "__main__":
    main()
