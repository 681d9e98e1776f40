"""Build the package's shared libraries in-tree with hipcc, for gfx950 only.

Usage: ``python -m exact_tiled_attention_13_amd.build`` (or call :func:`build`).

* ``libfa_mi355x.so`` -- the attention library (include/fa_mi355x.h);
* ``libfa_mi355x_ldspoison.so`` -- the same sources built with
  ``-DFA_LDS_POISON``: every kernel fills its LDS with NaN bit patterns
  before its first barrier, so that a read of LDS that no load or store
  wrote shows up as NaN in the results (a race check for the parity tests);
* ``libfa_micro.so`` -- microbenchmarks of the units the kernels depend on
  (include/fa_micro.h).

Each source compiles to an object under ``_build/`` in parallel, then one
``hipcc -shared`` link per library writes it into the package directory.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa_mi355x.so")
LIB_POISON = os.path.join(PKG, "libfa_mi355x_ldspoison.so")
LIB_MICRO = os.path.join(PKG, "libfa_micro.so")

SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_fp32.hip", "fwd_fp8.hip", "bwd_bf16.hip", "decode_bf16.hip",
           "noalloc.hip"]
MICRO_SOURCES = ["micro.hip"]

# (library, sources, extra defines, object-name suffix)
TARGETS = [
    (LIB, SOURCES, (), ""),
    (LIB_POISON, SOURCES, ("-DFA_LDS_POISON=1",), "_ldspoison"),
    (LIB_MICRO, MICRO_SOURCES, (), ""),
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # Packed-fp32 VALU forms are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# The backward dK/dV kernel runs one wave per SIMD with more live state than
# 256 VGPRs; by default every MFMA of such a kernel writes AGPRs, and the
# softmax then copies S and dP back to VGPRs each tile. The VGPR form keeps
# S / dP in VGPRs (the accumulators that do not fit spill to AGPRs instead).
EXTRA_FLAGS = {"bwd_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
               "decode_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
               "fwd_fp8.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(job) -> str:
    src, defines, suffix = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC, *FLAGS, *defines, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o",
           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _check_stubs(lib: str) -> None:
    """Fail if the host side of any kernel launch was left undefined.

    hipcc can drop a kernel template's host launch stub without an error (a
    device-only construct that the host pass rejects silently); the library
    then links but fails to load. nm lists such stubs as undefined."""
    r = subprocess.run(["nm", "-C", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{r.stderr}")
    missing = [ln.strip() for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the host code:\n" + "\n".join(missing))


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_stubs(tmp)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source of every library and link them. Returns the attention library's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, defines, suffix) for _, srcs, defines, suffix in TARGETS for src in srcs]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = dict(zip(jobs, ex.map(_compile, jobs)))
    for lib, srcs, defines, suffix in TARGETS:
        _link(lib, [objs[(src, defines, suffix)] for src in srcs])
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
