"""Microbenchmarks of the MI355X units the attention kernels depend on.

ctypes binding of ``libfa_micro.so`` (C ABI in include/fa_micro.h) plus the
arithmetic that turns its event times and clock stamps into rates. Each
result states the shader clock the chip held while it ran (from the kernel's
own s_memtime / s_memrealtime stamps), so that a rate can be read against
the clock-derived peak.

``python -m exact_tiled_attention_13_amd.micro`` runs all of them and prints
one JSON object.
"""

from __future__ import annotations

import ctypes
import json
import os
import threading

import torch

LIB_MICRO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_micro.so")

FLOP_PER_MFMA_32x32x16 = 2 * 32 * 32 * 16
REALTIME_HZ = 100e6                     # s_memrealtime counts at a constant 100 MHz

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_MICRO):
                raise RuntimeError(f"{LIB_MICRO} is missing: build it with `python -m exact_tiled_attention_13_amd.build`")
            L = ctypes.CDLL(LIB_MICRO)
            vp, ci, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
            L.fa_micro_mfma_bf16.argtypes = [vp, vp, ci, ci, ci, vp]
            L.fa_micro_exp2.argtypes = [vp, vp, ci, ci, vp]
            L.fa_micro_mfma_valu.argtypes = [vp, vp, ci, ci, ci, ci, vp]
            L.fa_micro_mfma_valu.restype = ci
            L.fa_micro_fp8_dot.argtypes = [vp, vp, vp, ci, ci, vp]
            L.fa_micro_atomic_add.argtypes = [vp, ll, ci, vp]
            for f in (L.fa_micro_mfma_bf16, L.fa_micro_exp2, L.fa_micro_fp8_dot, L.fa_micro_atomic_add):
                f.restype = ci
            _lib = L
        return _lib


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _timed(dev, launch, reps: int = 3):
    """Run launch() once untimed, then `reps` times between HIP events; returns the fastest run in ms."""
    if launch() != 0:
        raise RuntimeError("microbenchmark launch rejected")
    torch.cuda.synchronize(dev)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if launch() != 0:
            raise RuntimeError("microbenchmark launch rejected")
        e1.record()
        torch.cuda.synchronize(dev)
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    return best


def clock_ghz(clk: torch.Tensor) -> float:
    """Median over workgroups of (shader-clock ticks / real-time ticks) x 100 MHz, from [blocks, 4] stamps."""
    c = clk.view(-1, 4).cpu().to(torch.float64)
    dt, dr = c[:, 1] - c[:, 0], c[:, 3] - c[:, 2]
    ok = dr > 0
    return float((dt[ok] / dr[ok]).median()) * REALTIME_HZ / 1e9


def mfma_bf16(dev=None, blocks_per_cu: int = 4, iters: int = 40000, reps: int = 3, mode: int = 0) -> dict:
    """Sustained v_mfma_f32_32x32x16_bf16 rate with every CU busy (four waves per SIMD, four independent
    accumulators per wave). Returns TFLOP/s, the shader clock during the run, and the rate the clock implies
    at one MFMA per 32 clocks per SIMD (MI355X's 1024 dense bf16 FLOP per clock per SIMD). `mode` picks the
    operand source (include/fa_micro.h): 0 constant registers, 1 changing pseudo-random registers,
    2 the A operand from LDS, 3 both operands from LDS (the LDS modes hold 64 KB per workgroup, so two
    workgroups share a CU: two waves per SIMD), 4 / 5 as 1 with one / two accumulator chains per wave."""
    dev = dev or torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * blocks_per_cu
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    ms = _timed(dev, lambda: lib().fa_micro_mfma_bf16(out.data_ptr(), clk.data_ptr(), blocks, iters, mode, _stream(dev)),
                reps)
    flop = blocks * 4.0 * iters * 4 * FLOP_PER_MFMA_32x32x16
    ghz = clock_ghz(clk)
    tflops = flop / ms / 1e9
    at_clock = cus * 4 * 1024 * ghz * 1e9 / 1e12
    return {"mode": mode, "tflops": round(tflops, 1), "clock_ghz": round(ghz, 3), "ms": round(ms, 3),
            "peak_at_clock_tflops": round(at_clock, 1), "util_at_clock": round(tflops / at_clock, 4),
            "cus": cus, "blocks": blocks, "iters": iters}


def mfma_with_valu(dev=None, nfma: int = 0, nexp: int = 0, iters: int = 20000, reps: int = 3,
                   waves_per_simd: int = 2) -> dict:
    """MFMA rate when each MFMA of a wave is followed by `nfma` v_fma_f32 and `nexp` v_exp_f32 of its own
    (random operands; `waves_per_simd` workgroups of four waves per CU): how much VALU work a wave can place
    between its MFMAs for free, with or without a second wave on its SIMD."""
    dev = dev or torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * waves_per_simd
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    ms = _timed(dev, lambda: lib().fa_micro_mfma_valu(out.data_ptr(), clk.data_ptr(), blocks, iters, nfma, nexp,
                                                      _stream(dev)), reps)
    flop = blocks * 4.0 * iters * 4 * FLOP_PER_MFMA_32x32x16
    ghz = clock_ghz(clk)
    tflops = flop / ms / 1e9
    at_clock = cus * 4 * 1024 * ghz * 1e9 / 1e12
    return {"nfma": nfma, "nexp": nexp, "waves_per_simd": waves_per_simd, "tflops": round(tflops, 1),
            "clock_ghz": round(ghz, 3),
            "util_at_clock": round(tflops / at_clock, 4), "ms": round(ms, 3)}


def exp2_rate(dev=None, blocks_per_cu: int = 4, iters: int = 20000, reps: int = 3) -> dict:
    """Issue rate of v_exp_f32 (eight independent chains per lane): clocks per wave instruction per SIMD."""
    dev = dev or torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * blocks_per_cu
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    ms = _timed(dev, lambda: lib().fa_micro_exp2(out.data_ptr(), clk.data_ptr(), blocks, iters, _stream(dev)), reps)
    ghz = clock_ghz(clk)
    instr_per_simd = blocks * 4 * iters * 8 / (cus * 4)
    clocks = ms * 1e-3 * ghz * 1e9
    return {"clocks_per_wave_instr": round(clocks / instr_per_simd, 2), "clock_ghz": round(ghz, 3),
            "ms": round(ms, 3), "blocks": blocks, "iters": iters}


def fp8_dot(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """C[p] = sum_s A[p, s] B[p, s]^T on the FP8 matrix cores. a, b: uint8 E4M3 codes [P, chain, 32, 64] on the
    GPU (b holds the columns of each B_s as rows). Returns fp32 [P, 32, 32]."""
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or a.shape != b.shape or a.dim() != 4 \
            or tuple(a.shape[2:]) != (32, 64) or not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a, b: contiguous uint8 [P, chain, 32, 64] of equal shape")
    P, chain = int(a.shape[0]), int(a.shape[1])
    c = torch.empty((P, 32, 32), dtype=torch.float32, device=a.device)
    st = lib().fa_micro_fp8_dot(a.data_ptr(), b.data_ptr(), c.data_ptr(), P, chain, _stream(a.device))
    if st != 0:
        raise RuntimeError(f"fa_micro_fp8_dot rejected its arguments ({st})")
    return c


def atomic_add(dev=None, n: int = 1 << 26, reps: int = 4) -> dict:
    """Throughput of coalesced fp32 global atomic adds (bytes = 4 n reps)."""
    dev = dev or torch.device("cuda:0")
    buf = torch.zeros(n, dtype=torch.float32, device=dev)
    ms = _timed(dev, lambda: lib().fa_micro_atomic_add(buf.data_ptr(), n, reps, _stream(dev)))
    return {"gbs": round(4.0 * n * reps / ms / 1e6, 1), "ms": round(ms, 3), "n": n, "reps": reps}


def main():
    dev = torch.device("cuda:0")
    res = {f"mfma_bf16_mode{m}": mfma_bf16(dev, mode=m) for m in (0, 1, 2, 3, 4, 5)}
    res.update({"exp2": exp2_rate(dev), "atomic_add_f32": atomic_add(dev)})
    res["mfma_with_valu"] = [mfma_with_valu(dev, f, e) for f, e in ((0, 0), (2, 0), (4, 0), (8, 0), (0, 1), (0, 2),
                                                                    (0, 4), (4, 2), (6, 2))]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
