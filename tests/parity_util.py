"""Helpers shared by the GPU parity tests: error metric, tolerances, sampling.

The error of a tensor is max|T_gpu - T_ref| / max|T_ref| over the whole tensor
(or over the sampled elements), where T_ref is the fp64 oracle's value on the
same inputs. Tolerances: bf16 inputs with fp32 accumulation, O <= 2e-2 and
dQ, dK, dV <= 5e-2; the fp32 forward <= 1e-4. LSE is compared in absolute
terms: it is formed from exactly-representable products summed in fp32, so
<= 1e-3 for bf16 and <= 1e-5 for fp32.
"""

import numpy as np
import torch

TOL_O_BF16 = 2e-2
TOL_GRAD_BF16 = 5e-2
TOL_O_FP32 = 1e-4
TOL_LSE_BF16 = 1e-3
TOL_LSE_FP32 = 1e-5

DEV = "cuda:0"


def nerr(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values in the GPU result"
    denom = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (denom if denom > 0 else 1.0))


def aerr(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values in the GPU result"
    return float(np.abs(got - ref).max())


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Rows that cover tile edges (multiples of 32/64/128 and their neighbours),
    both ends of the sequence, and random interior rows."""
    fixed = {0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 65,
             N - 64, N - 33, N - 32, N - 2, N - 1}
    fixed = {r for r in fixed if 0 <= r < N}
    rng = np.random.default_rng(seed)
    extra = rng.choice(N, size=min(N, max(0, count - len(fixed))), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)), dtype=np.int64)
