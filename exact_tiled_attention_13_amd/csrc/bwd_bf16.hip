// bwd_bf16.hip -- bf16 backward of exact tiled attention for gfx950.
//
// The pages say only that gradients, like outputs, match exact attention
// within a tolerance (page "FlashAttention-2: atención eficiente en GPU para
// contextos largos", section "Bloques pequeños, normalización global"). The
// gradients computed here are the textbook chain rule through the row
// softmax, with P recomputed tile by tile from Q, K and the forward's LSE so
// that no N x N matrix is stored:
//
//     D_i = dO_i . O_i                      (kernel bwd_pre)
//     P   = exp(scale * Q K^T - LSE)         (masked entries 0)
//     dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
//     dK  = scale * dS^T Q                  (kernel bwd_dkdv: key-block outer)
//     dQ  = scale * dS K                    (kernel bwd_dq: query-block outer)
//
// dK/dV and dQ are produced by two separate kernels, each owning its output
// rows, so there are no atomics and the result is bitwise deterministic. The
// price is recomputing S and dP in the dQ kernel (7 products instead of 5).
// The same work split as the forward applies: the grid covers (row block,
// head, batch), every wavefront owns 32 rows of the output it accumulates,
// and causal tiles that are entirely masked are skipped.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {

// D_i = sum_c dO[b,i,h,c] * O[b,i,h,c] in fp32, written as [B, H, N].
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
    constexpr int TPR = D / 8;               // threads per row (8 elements each)
    constexpr int RPB = 256 / TPR;           // rows per block
    const long long rows = (long long)a.B * a.N * a.H;
    const long long r = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float acc = 0.f;
    if (r < rows) {
        const u32x4 o = ld16(static_cast<const __bf16*>(a.o) + r * D + c * 8);
        const u32x4 g = ld16(static_cast<const __bf16*>(a.dO) + r * D + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += __uint_as_float(o[w] << 16) * __uint_as_float(g[w] << 16);
            acc += __uint_as_float(o[w] & 0xffff0000u) * __uint_as_float(g[w] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (r < rows && c == 0) {
        const long long h = r % a.H;
        const long long n = (r / a.H) % a.N;
        const long long b = r / ((long long)a.H * a.N);
        a.dd[(b * a.H + h) * a.N + n] = acc;
    }
}

// Stage a block of 4 rows x 8 columns (rows row0..row0+3 of a [*, rs] bf16
// matrix, columns col..col+7) from global memory; rows >= nrows read as 0.
__device__ __forceinline__ void load_4x8(u32x4 (&r)[4], const __bf16* g, size_t rs, int row0, int nrows, int col) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = (row0 + i < nrows) ? ld16(g + (size_t)(row0 + i) * rs + col) : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys (4 waves x 32 keys), loop over query
// tiles of 64 rows staged in LDS both row-major (for S = Q K^T, dP = dO V^T)
// and transposed (for dV^T += dO^T P and dK^T += Q^T dS).
//
// In the 32x32 accumulators of S = Q K^T and dP = dO V^T each lane holds one
// key column (lane % 32) and 16 query rows, which is exactly the B operand
// layout dV^T = dO^T P and dK^T = Q^T dS need (queries permuted within each
// 16-row chunk in the transposed tiles, see kperm4).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int BK = 128;              // keys per workgroup
    constexpr int BQ = 64;               // queries per tile
    constexpr int RS_ = D + 8;           // row-major tile stride
    constexpr int TS = BQ + 8;           // transposed tile stride
    constexpr int R_ELEMS = BQ * RS_;
    constexpr int T_ELEMS = D * TS;
    constexpr int STAGE = 2 * R_ELEMS + 2 * T_ELEMS + 2 * BQ * 2;  // Q, dO, Q^T, dO^T, lse2, D (as bf16 slots)
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int MB = BQ / 32;          // 32-query blocks per tile
    constexpr int STAGERS = BQ / 4 * (D / 8);  // threads holding a 4x8 block

    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

    const int B = a.B, H = a.H, N = a.N;
    const int nk = (N + BK - 1) / BK;
    const int r = xcd_remap(blockIdx.x, nk * B * H);
    const int bh = r / nk;
    const int kb = r - bh * nk;         // causal: every key block visits the same tail, order kept
    const int b = bh / H, h = bh - b * H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;
    const size_t base = ((size_t)b * N * H + h) * D;
    const __bf16* Qg = static_cast<const __bf16*>(a.q) + base;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + base;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + base;
    const __bf16* dOg = static_cast<const __bf16*>(a.dO) + base;
    const float* lseg = a.lse + (size_t)bh * N;
    const float* ddg = a.dd + (size_t)bh * N;

    const int k0 = kb * BK;
    const int kw = k0 + wave * 32;       // first key of this wave
    const int myk = kw + l32;            // key column owned by this lane

    // K and V as B operands (lane holds row myk, d chunk c*16 + hi*8 .. +8).
    bf16x8 kf[DC], vf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (myk < N) {
            kv = ld16(Kg + (size_t)myk * rs + c * 16 + hi * 8);
            vv = ld16(Vg + (size_t)myk * rs + c * 16 + hi * 8);
        }
        kv ^= a.qsign;  // negative scale folded into S's operand
        kf[c] = as_bf16x8(kv);
        vf[c] = as_bf16x8(vv);
    }

    f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        dvacc[i] = f32x16{};
        dkacc[i] = f32x16{};
    }

    const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
    const int ntiles = (N - qstart + BQ - 1) / BQ;
    const float c2 = a.c2;

    // staging map: thread -> (query group of 4 rows, d group of 8 columns)
    const int sg = tid % (BQ / 4);
    const int sd = tid / (BQ / 4);
    u32x4 qr[4], gr[4];
    float lr = 0.f, dr = 0.f;

    auto load_tile = [&](int t) {
        const int q0 = qstart + t * BQ;
        if (tid < STAGERS) {
            load_4x8(qr, Qg, rs, q0 + sg * 4, N, sd * 8);
            load_4x8(gr, dOg, rs, q0 + sg * 4, N, sd * 8);
        }
        if (tid < BQ) {
            const int q = q0 + tid;
            lr = (q < N) ? lseg[q] * kLog2e : INFINITY;   // padded rows: P = 0
            dr = (q < N) ? ddg[q] : 0.f;
        }
    };
    auto store_tile = [&](int stage) {
        __bf16* Qs = smem + stage * STAGE;
        __bf16* Gs = Qs + R_ELEMS;
        __bf16* Qt = Gs + R_ELEMS;
        __bf16* Gt = Qt + T_ELEMS;
        float* Ls = reinterpret_cast<float*>(Gt + T_ELEMS);
        float* Ds = Ls + BQ;
        if (tid < STAGERS) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                st16(Qs + (sg * 4 + i) * RS_ + sd * 8, qr[i]);
                st16(Gs + (sg * 4 + i) * RS_ + sd * 8, gr[i]);
            }
            u32x2 cq[8], cg[8];
            transpose_4x8(qr, cq);
            transpose_4x8(gr, cg);
            const int pos = kperm4(sg * 4);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st8(Qt + (sd * 8 + c) * TS + pos, cq[c]);
                st8(Gt + (sd * 8 + c) * TS + pos, cg[c]);
            }
        }
        if (tid < BQ) {
            Ls[tid] = lr;
            Ds[tid] = dr;
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int q0 = qstart + t * BQ;
        if (t + 1 < ntiles) load_tile(t + 1);
        const __bf16* Qs = smem + (t & 1) * STAGE;
        const __bf16* Gs = Qs + R_ELEMS;
        const __bf16* Qt = Gs + R_ELEMS;
        const __bf16* Gt = Qt + T_ELEMS;
        const float* Ls = reinterpret_cast<const float*>(Gt + T_ELEMS);
        const float* Ds = Ls + BQ;

        // Causal: the tile's last query precedes this wave's first key.
        const bool active = !CAUSAL || (q0 + BQ - 1 >= kw);
        if (active) {
            const bool masked = CAUSAL && (q0 < kw + 31);
            bf16x8 pb[BQ / 16], sb[BQ / 16];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (mb * 32 + l32) * RS_ + c * 16 + hi * 8);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[c], s, 0, 0, 0);
                }
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8 ga = *reinterpret_cast<const bf16x8*>(Gs + (mb * 32 + l32) * RS_ + c * 16 + hi * 8);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[c], dp, 0, 0, 0);
                }
                float p[16], ds[16];
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ql = mb * 32 + 8 * g4 + 4 * hi;   // tile-local query of element 4*g4
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + ql);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int u = 4 * g4 + e;
                        float pv = exp2_fast(__builtin_fmaf(s[u], c2, -l4[e]));
                        if (masked && myk > q0 + ql + e) pv = 0.f;
                        p[u] = pv;
                        ds[u] = pv * (dp[u] - d4[e]);
                    }
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    u32x4 wp, wd;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wp[e] = pack_bf16x2(p[half * 8 + 2 * e], p[half * 8 + 2 * e + 1]);
                        wd[e] = pack_bf16x2(ds[half * 8 + 2 * e], ds[half * 8 + 2 * e + 1]);
                    }
                    pb[mb * 2 + half] = as_bf16x8(wp);
                    sb[mb * 2 + half] = as_bf16x8(wd);
                }
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int qc = 0; qc < BQ / 16; ++qc) {
                    const bf16x8 ga = *reinterpret_cast<const bf16x8*>(Gt + (db * 32 + l32) * TS + qc * 16 + hi * 8);
                    dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pb[qc], dvacc[db], 0, 0, 0);
                    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qt + (db * 32 + l32) * TS + qc * 16 + hi * 8);
                    dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb[qc], dkacc[db], 0, 0, 0);
                }
            }
        }

        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    if (myk < N) {
        __bf16* dkrow = static_cast<__bf16*>(a.dk) + base + (size_t)myk * rs;
        __bf16* dvrow = static_cast<__bf16*>(a.dv) + base + (size_t)myk * rs;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hi;
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[db][4 * g] * sc, dkacc[db][4 * g + 1] * sc);
                wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * sc, dkacc[db][4 * g + 3] * sc);
                wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                st8(dkrow + d0, wk);
                st8(dvrow + d0, wv);
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries (4 waves x 32), loop over key tiles staged
// in LDS row-major (K for S^T = K Q^T, V for dP^T = V dO^T) and transposed
// (K^T for dQ^T += K^T dS^T). The accumulators hold one query per lane, as
// in the forward.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
    constexpr int BM = 128;
    constexpr int BN = 8192 / D;         // keys per tile
    constexpr int RS_ = D + 8;
    constexpr int TS = BN + 8;
    constexpr int R_ELEMS = BN * RS_;
    constexpr int T_ELEMS = D * TS;
    constexpr int STAGE = 2 * R_ELEMS + T_ELEMS;   // K, V, K^T
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int KB = BN / 32;
    constexpr int NKG = BN / 4;
    static_assert(NKG * (D / 8) == 256, "staging assumes 256 threads x (4 keys x 8 d)");

    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

    const int B = a.B, H = a.H, N = a.N;
    const int nq = (N + BM - 1) / BM;
    const int r = xcd_remap(blockIdx.x, nq * B * H);
    const int bh = r / nq;
    int qb = r - bh * nq;
    if (CAUSAL) qb = nq - 1 - qb;
    const int b = bh / H, h = bh - b * H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;
    const size_t base = ((size_t)b * N * H + h) * D;
    const __bf16* Qg = static_cast<const __bf16*>(a.q) + base;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + base;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + base;
    const __bf16* dOg = static_cast<const __bf16*>(a.dO) + base;

    const int q0 = qb * BM;
    const int qw = q0 + wave * 32;
    const int myq = qw + l32;

    bf16x8 qf[DC], gf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        u32x4 qv = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
        if (myq < N) {
            qv = ld16(Qg + (size_t)myq * rs + c * 16 + hi * 8);
            gv = ld16(dOg + (size_t)myq * rs + c * 16 + hi * 8);
        }
        qv ^= a.qsign;
        qf[c] = as_bf16x8(qv);
        gf[c] = as_bf16x8(gv);
    }
    const float lse2 = (myq < N) ? a.lse[(size_t)bh * N + myq] * kLog2e : 0.f;
    const float dd = (myq < N) ? a.dd[(size_t)bh * N + myq] : 0.f;

    f32x16 dqacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dqacc[i] = f32x16{};

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;
    const float c2 = a.c2;

    const int skg = tid % NKG;
    const int sdg = tid / NKG;
    u32x4 kr[4], vr[4];
    auto load_tile = [&](int t) {
        const int j0 = t * BN;
        load_4x8(kr, Kg, rs, j0 + skg * 4, N, sdg * 8);
        load_4x8(vr, Vg, rs, j0 + skg * 4, N, sdg * 8);
    };
    auto store_tile = [&](int stage) {
        __bf16* Ks = smem + stage * STAGE;
        __bf16* Vs = Ks + R_ELEMS;
        __bf16* Kt = Vs + R_ELEMS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st16(Ks + (skg * 4 + i) * RS_ + sdg * 8, kr[i]);
            st16(Vs + (skg * 4 + i) * RS_ + sdg * 8, vr[i]);
        }
        u32x2 ck[8];
        transpose_4x8(kr, ck);
        const int pos = kperm4(skg * 4);
#pragma unroll
        for (int c = 0; c < 8; ++c) st8(Kt + (sdg * 8 + c) * TS + pos, ck[c]);
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * BN;
        if (t + 1 < ntiles) load_tile(t + 1);
        const __bf16* Ks = smem + (t & 1) * STAGE;
        const __bf16* Vs = Ks + R_ELEMS;
        const __bf16* Kt = Vs + R_ELEMS;

        const bool active = !CAUSAL || (j0 <= qw + 31);
        if (active) {
            const bool masked = (CAUSAL && j0 + BN - 1 > qw) || (j0 + BN > N);
            bf16x8 sb[BN / 16];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + l32) * RS_ + c * 16 + hi * 8);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s, 0, 0, 0);
                }
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vs + (kb * 32 + l32) * RS_ + c * 16 + hi * 8);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[c], dp, 0, 0, 0);
                }
                float ds[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    float pv = exp2_fast(__builtin_fmaf(s[u], c2, -lse2));
                    if (masked) {
                        const int key = j0 + kb * 32 + 8 * (u >> 2) + 4 * hi + (u & 3);
                        if (key >= N || (CAUSAL && key > myq)) pv = 0.f;
                    }
                    ds[u] = pv * (dp[u] - dd);
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(ds[half * 8 + 2 * e], ds[half * 8 + 2 * e + 1]);
                    sb[kb * 2 + half] = as_bf16x8(w);
                }
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int kc = 0; kc < BN / 16; ++kc) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kt + (db * 32 + l32) * TS + kc * 16 + hi * 8);
                    dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sb[kc], dqacc[db], 0, 0, 0);
                }
        }

        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    if (myq < N) {
        __bf16* row = static_cast<__bf16*>(a.dq) + base + (size_t)myq * rs;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(dqacc[db][4 * g] * sc, dqacc[db][4 * g + 1] * sc);
                w[1] = pack_bf16x2(dqacc[db][4 * g + 2] * sc, dqacc[db][4 * g + 3] * sc);
                st8(row + db * 32 + 8 * g + 4 * hi, w);
            }
    }
}

template <int D>
static hipError_t launch_prep(const BwdArgs& a, hipStream_t stream) {
    const long long rows = (long long)a.B * a.N * a.H;
    const long long rpb = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
    const long long g = (long long)((a.N + 127) / 128) * a.B * a.H;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)g), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
    const long long g = (long long)((a.N + 127) / 128) * a.B * a.H;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)g), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, int d, hipStream_t stream) {
    return d == 128 ? launch_prep<128>(a, stream) : launch_prep<64>(a, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch_dkdv<128, true>(a, stream) : launch_dkdv<128, false>(a, stream);
    return causal ? launch_dkdv<64, true>(a, stream) : launch_dkdv<64, false>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch_dq<128, true>(a, stream) : launch_dq<128, false>(a, stream);
    return causal ? launch_dq<64, true>(a, stream) : launch_dq<64, false>(a, stream);
}

}  // namespace fa
