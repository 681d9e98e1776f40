"""FP8 (e4m3) forward: the e4m3 rounding and the tiled algorithm with 8-bit P.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

Source: page "FlashAttention-T: Optimización GPU para LLMs Escalables",
sections "Innovaciones técnicas frente a FlashAttention original" and the
performance table: the method supports 8-bit (FP8) quantisation on recent
GPUs. The page gives no algorithm. Readings used here:

* Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals, no infinities, largest finite value 448;
  conversions round to nearest, ties to even. (gfx950's matrix cores read
  this encoding.)
* Inputs are per-tensor quantised: the real values are q = Q8 * dq,
  k = K8 * dk, v = V8 * dv with e4m3 tensors Q8, K8, V8 and fp32 descales.
  Those dequantised values are the attention inputs; scores and softmax
  statistics are exact (fp32 on the GPU, fp64 here).
* The probabilities that multiply V are themselves 8-bit: key tiles of
  ``tile`` keys are processed in order with the online softmax of
  :mod:`oracle.online` (running max m over the tiles seen so far, rescale of
  the running sums by exp(m_old - m_new)); within a tile P = exp(S - m) <= 1
  is rounded to e4m3 before it multiplies V, while the row sum l uses the
  unrounded P. O = (sum of rescaled e4m3(P) V) / l, LSE = m + ln l.

With the rounding replaced by the identity this is exactly the online
softmax, i.e. exact attention; tests pin both facts.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def round_e4m3(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value, ties to even; |x| > 448 saturates to +-448.

    Written from the format: normal values have 3 fraction bits and exponents
    -6 .. 8; below 2^-6 the spacing is fixed at 2^-9 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    nz = a > 0
    _, ex = np.frexp(np.where(nz, a, 1.0))     # a = f * 2^ex with f in [0.5, 1): exponent ex - 1, exactly
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)   # subnormals share exponent -6's spacing
    quantum = np.exp2(e - 3.0)                 # spacing of representable values at this exponent
    q = a / quantum
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))
    r = r + up
    out = np.where(nz, r * quantum, 0.0)
    out = np.minimum(out, E4M3_MAX)
    return np.copysign(out, x)


def e4m3_values() -> np.ndarray:
    """All 254 finite E4M3 codes 0x00..0xFE except the NaN codes 0x7F / 0xFF, decoded in code order."""
    vals = []
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            continue                           # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(s * v)
    return np.array(vals)


def attn_fwd_fp8_head(q, k, v, causal: bool, scale: float, tile: int = 64, round_p=round_e4m3,
                      flip_eta: float | None = None):
    """One head: q [N, d], k [N, d], v [N, d] (dequantised values) -> (O [N, d], LSE [N]).

    With ``flip_eta`` set, also returns a bound [N, d] on how far O moves if
    every probability within a relative ``flip_eta`` of an E4M3 rounding
    boundary rounds to the other neighbour instead (an implementation that
    computes P with a relative error below flip_eta can only differ from
    this oracle in those roundings): the sum over such keys of
    |E4M3(P (1 + eta)) - E4M3(P (1 - eta))| |v|, rescaled to the final
    maximum and divided by l. ``flip_eta="fp32"`` derives eta per row for
    scores accumulated on the FP8 matrix cores (see fp32_p_error) and adds
    the error of evaluating the rest that way: MFMA_FP8_GAMMA_SCALE gamma_n
    sum_j E4M3(P_j) |v_j| / l for the P V sums, gamma_n |O| for the fp32 row
    sum l (n = N + 2 terms each), and eta |O| because l sums the unrounded P.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n = q.shape[0]
    s_all = scale * (q @ k.T)
    if causal:
        s_all = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], s_all, -np.inf)
    eta = fp32_p_error(q, k, scale) if isinstance(flip_eta, str) else flip_eta
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    flip = np.zeros_like(acc)
    accabs = np.zeros_like(acc)
    for t0 in range(0, n, tile):
        s = s_all[:, t0:t0 + tile]
        mt = s.max(axis=1)
        mn = np.maximum(m, mt)
        safe = np.where(np.isfinite(mn), mn, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        p = np.exp(s - safe[:, None])          # masked keys: exp(-inf) = 0
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + round_p(p) @ v[t0:t0 + tile]
        if flip_eta is not None:
            e_row = np.broadcast_to(np.asarray(eta, dtype=np.float64).reshape(-1, 1) if np.ndim(eta) else eta,
                                    p.shape)
            gap = np.abs(round_e4m3(p * (1 + e_row)) - round_e4m3(p * (1 - e_row)))
            flip = flip * alpha[:, None] + gap @ np.abs(v[t0:t0 + tile])
            accabs = accabs * alpha[:, None] + round_p(p) @ np.abs(v[t0:t0 + tile])
        m = mn
    o = acc / l[:, None]
    if flip_eta is not None:
        bound = flip / l[:, None]
        if isinstance(flip_eta, str):
            u = 2.0 ** -24
            g = (n + 2) * u / (1 - (n + 2) * u)
            # l sums the unrounded P, whose relative error (eta) reaches O unchanged.
            bound = bound + g * (MFMA_FP8_GAMMA_SCALE * accabs / l[:, None] + np.abs(o)) \
                + np.asarray(eta).reshape(-1, 1) * np.abs(o)
        return o, m + np.log(l), bound
    return o, m + np.log(l)


# Sums of products formed on gfx950's FP8 matrix cores err by more than a
# sequential fp32 sum: a probe of v_mfma_f32_32x32x64_f8f6f4 measured up to
# 2.3 gamma_64 sum |a_i b_i| (gamma_n = n u / (1 - n u), u = 2^-24). The bounds
# below scale gamma by this factor for such sums.
MFMA_FP8_GAMMA_SCALE = 8.0


def fp32_p_error(q, k, scale: float, gamma_scale: float = MFMA_FP8_GAMMA_SCALE) -> np.ndarray:
    """Per query row, a bound on the relative error of P = exp(S - m) when the scores are d-term dot products
    accumulated in fp32 (unit roundoff u = 2^-24; gamma scaled by ``gamma_scale`` for sums formed on the FP8
    matrix cores, 1 for a sequential fp32 sum) and scaled by an fp32 factor, and exp is evaluated in fp32.

    The standard bound |fl(sum a_i b_i) - sum a_i b_i| <= gamma_d sum |a_i b_i| (gamma_d = d u / (1 - d u))
    gives each score an absolute error e_j <= |scale| (gamma_d sum_i |q_i k_ji| + 4 u |sum_i q_i k_ji|); the
    exponent S_j - m then errs by at most 2 max_j e_j (m is itself one of the perturbed scores), and the
    fp32 exponential adds a few units: eta = exp(2 max_j e_j) (1 + 8 u) - 1.
    """
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    u = 2.0 ** -24
    dd = q.shape[1]
    gamma = dd * u / (1 - dd * u)
    e = abs(scale) * (gamma_scale * gamma * (np.abs(q) @ np.abs(k).T) + 4 * u * np.abs(q @ k.T))
    return np.expm1(2 * e.max(axis=1)) * (1 + 8 * u) + 8 * u


def attn_fwd_fp8(q8, k8, v8, dq: float, dk: float, dv: float, causal: bool, scale: float, tile: int = 64,
                 round_p=round_e4m3, flip_eta: float | None = None):
    """q8, k8, v8: e4m3 values (already representable) [B, N, H, d]; returns (O [B, N, H, d], LSE [B, H, N]),
    plus the rounding-flip bound [B, N, H, d] of attn_fwd_fp8_head when ``flip_eta`` is set."""
    q8, k8, v8 = (np.asarray(t, dtype=np.float64) for t in (q8, k8, v8))
    B, N, H, d = q8.shape
    o = np.empty((B, N, H, d))
    lse = np.empty((B, H, N))
    bound = np.zeros((B, N, H, d))
    for b in range(B):
        for h in range(H):
            r = attn_fwd_fp8_head(q8[b, :, h] * dq, k8[b, :, h] * dk, v8[b, :, h] * dv, causal, scale, tile,
                                  round_p, flip_eta)
            o[b, :, h], lse[b, h] = r[0], r[1]
            if flip_eta is not None:
                bound[b, :, h] = r[2]
    if flip_eta is not None:
        return o, lse, bound
    return o, lse


def quantize_e4m3(x, amax_target: float = E4M3_MAX):
    """Per-tensor quantisation of real values: descale = amax / 448, values = round_e4m3(x / descale).

    Returns (e4m3 values as float64, descale as a Python float, exactly representable in fp32).
    """
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.abs(x).max())
    ds = float(np.float32(amax / amax_target)) if amax > 0 else 1.0
    return round_e4m3(x / ds), ds


def flops_fwd_fp8(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Counted FLOP as for the bf16 forward: 4*B*H*N^2*d, halved under causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


__all__ = ["E4M3_MAX", "round_e4m3", "e4m3_values", "attn_fwd_fp8_head", "attn_fwd_fp8", "quantize_e4m3",
           "flops_fwd_fp8", "fp32_p_error"]
