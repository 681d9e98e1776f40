// bwd_bf16.hip -- bf16 backward of exact tiled attention for gfx950.
//
// The pages say only that gradients, like outputs, match exact attention
// within a tolerance (page "FlashAttention-2: atención eficiente en GPU para
// contextos largos", section "Bloques pequeños, normalización global"). The
// gradients computed here are the textbook chain rule through the row
// softmax, with P recomputed tile by tile from Q, K and the forward's LSE so
// that no N x N matrix is stored:
//
//     D_i = dO_i . O_i                      (kernel bwd_pre, or bwd_dq with PREP)
//     P   = exp(scale * Q K^T - LSE)         (masked entries 0)
//     dV  = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
//     dK  = scale * dS^T Q                  (kernel bwd_dkdv: key-block outer)
//     dQ  = scale * dS K                    (kernel bwd_dq: query-block outer)
//
// dK/dV and dQ are produced by two separate kernels, each owning its output
// rows, so there are no atomics and the result is bitwise deterministic (fp32
// atomics on this chip sustain far less than the dQ accumulation traffic). The
// price is recomputing S and dP in the dQ kernel (7 products instead of 5).
// The same work split as the forward applies: the grid covers (row block,
// head, batch), every wavefront owns 32 rows of the output it accumulates,
// and causal tiles that are entirely masked are skipped.
//
// Workspace: two fp32 arrays [B, H, Npad] (Npad = 64 * ceil(N / 64)), first
// -D_i, then LSE_i * log2(e); padded rows hold D = 0 and LSE = +inf, so their
// probabilities are exactly 0.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace fa {

// -D_i = -sum_c dO[b,i,h,c] * O[b,i,h,c] and LSE_i * log2(e), fp32 [B, H, Npad].
// D is stored negated so that the dK/dV kernel can start its dP accumulator
// at -D (dP - D then comes out of the MFMAs) and the dQ kernel adds it.
// One workgroup per 64-row block of one head: D/8 threads reduce a row (16
// bytes of O and dO each), the row results gather in LDS, and each statistic
// leaves as one contiguous 256-byte run (rows of one head are contiguous in
// the [B, H, Npad] arrays; per-row 4-byte stores strided by Npad would write
// whole memory sectors for 4 bytes each).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
    constexpr int TPR = D / 8;               // threads per row (8 elements each)
    constexpr int RPP = 256 / TPR;           // rows per pass
    constexpr int ROWS = 64;                 // rows per workgroup
    __shared__ float dsh[ROWS];
    lds_poison(dsh, sizeof(dsh));
    const int npad = (a.N + 63) & ~63;
    const int nblk = npad / ROWS;
    const int blk = blockIdx.x % nblk;
    const int bh = blockIdx.x / nblk;        // b * H + h
    const int b = bh / a.H, h = bh - b * a.H;
    const int c = threadIdx.x % TPR;
#pragma unroll
    for (int p = 0; p < ROWS / RPP; ++p) {
        const int rl = p * RPP + threadIdx.x / TPR;
        const int n = blk * ROWS + rl;
        float acc = 0.f;
        if (n < a.N) {
            const size_t src = (((size_t)b * a.N + n) * a.H + h) * D + c * 8;
            const u32x4 o = ld16(static_cast<const __bf16*>(a.o) + src);
            const u32x4 g = ld16(static_cast<const __bf16*>(a.dO) + src);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc += __uint_as_float(o[w] << 16) * __uint_as_float(g[w] << 16);
                acc += __uint_as_float(o[w] & 0xffff0000u) * __uint_as_float(g[w] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (c == 0) dsh[rl] = acc;
    }
    __syncthreads();
    if (threadIdx.x < ROWS) {
        const int n = blk * ROWS + threadIdx.x;
        const size_t i = (size_t)bh * npad + n;
        const bool real = n < a.N;
        a.dd[i] = real ? -dsh[threadIdx.x] : 0.f;
        a.lse2[i] = real ? a.lse[(size_t)bh * a.N + n] * kLog2e : INFINITY;
    }
}

// ---------------------------------------------------------------------------
// dK, dV for d = 64: one workgroup of 4 waves per 128 keys (32 per wave, K
// and V rows in VGPRs; two workgroups share a CU), looping over query tiles
// of 64 rows staged in LDS by direct loads.
//
// S = Q K^T and dP = dO V^T use row reads of the Q / dO tiles; in their 32x32
// accumulators each lane holds one key column (lane % 32) and 16 query rows,
// which is exactly the B operand layout of dV^T += dO^T P and dK^T += Q^T dS,
// whose A operands come from transposing reads of the same tiles.
template <int D, bool CAUSAL, bool GQA>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
    using T = LdsTile<D>;
    constexpr int NW = 4;
    constexpr int BK = NW * 32;          // keys per workgroup
    constexpr int BQ = T::ROWS;          // queries per tile
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int MB = BQ / 32;          // 32-query blocks per tile
    constexpr int RB = T::RB;
    constexpr int STAGE = 2 * T::BYTES + 2 * BQ * 4;   // Q, dO, lse2, dd

    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
    lds_poison(smem, sizeof(smem));

    const int B = a.B, H = a.H, N = a.N;
    const int npad = (N + 63) & ~63;
    const int Hkv = GQA ? a.Hkv : H;
    const int G = GQA ? H / Hkv : 1;     // query heads sharing this K/V head
    // Grouped-query split: the G heads run as S workgroups of GS heads each,
    // which write fp32 partial sums (reduced by bwd_dkdv_reduce_kernel).
    const int S = GQA ? a.gsplit : 1;
    const int GS = G / S;
    const int nk = (N + BK - 1) / BK;
    int unit, kb;                        // causal: low key blocks see the most query tiles, so go first
    work_item(blockIdx.x, nk, B * Hkv * S, CAUSAL, unit, kb);
    const int bhk = GQA ? unit / S : unit;
    const int sp = GQA ? unit - bhk * S : 0;   // part of the head group
    const int b = bhk / Hkv, hk = bhk - b * Hkv;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;                  // Q / dO row stride
    const size_t rskv = (size_t)Hkv * D;              // K / V / dK / dV row stride
    const size_t kvbase = ((size_t)b * N * Hkv + hk) * D;
    // Query head g of this workgroup's part is h = hk * G + sp * GS + g: its
    // Q / dO start D elements after head g - 1's, its statistics npad floats after.
    const size_t qbase = ((size_t)b * N * H + (size_t)hk * G + (size_t)sp * GS) * D;
    const __bf16* Qg0 = static_cast<const __bf16*>(a.q) + qbase;
    const __bf16* dOg0 = static_cast<const __bf16*>(a.dO) + qbase;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + kvbase;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + kvbase;
    const size_t stat0 = ((size_t)b * H + (size_t)hk * G + (size_t)sp * GS) * npad;

    const int k0 = kb * BK;
    const int kw = k0 + wave * 32;       // first key of this wave
    const int myk = kw + l32;            // key column owned by this lane

    // K and V rows as B operands (lane holds row myk, d chunk c*16 + hi*8 .. +8).
    bf16x8 kf[DC], vf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (myk < N) {
            kv = ld16(Kg + (size_t)myk * rskv + c * 16 + hi * 8);
            vv = ld16(Vg + (size_t)myk * rskv + c * 16 + hi * 8);
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

    const int qstart = CAUSAL ? k0 : 0;  // k0 is a multiple of BQ
    const int ntiles = (N - qstart + BQ - 1) / BQ;
    const float c2 = a.c2;
    const int rowb = T::rowbase(lane);
    const int trb0 = T::trbase(lane, 0);
    const int trb1 = T::trbase(lane, 1);

    auto stage_ptr = [&](int s) { return smem + s * STAGE; };
    unsigned toff[T::NINST / NW];
    T::template offsets<NW>(toff, rs, wave, lane);
    // Stage s receives query tile t of group head g.
    const uint32_t qspan = T::span(rs, N);
    auto dma = [&](int g, int t, int s) {
        unsigned char* st = stage_ptr(s);
        const int q0 = qstart + t * BQ;
        if (GQA && g > 0) {
            T::template load<NW>(st, Qg0 + (size_t)g * D, rs, q0, N, wave, lane, toff);
            T::template load<NW>(st + T::BYTES, dOg0 + (size_t)g * D, rs, q0, N, wave, lane, toff);
        } else {
            T::template load_buf<NW>(st, Qg0, qspan, rs, q0, N, wave, lane, toff);
            T::template load_buf<NW>(st + T::BYTES, dOg0, qspan, rs, q0, N, wave, lane, toff);
        }
        // q0 + 63 < npad: the padded statistics need no clamp.
        const size_t so = stat0 + (size_t)g * npad + q0 + lane;
        if (wave == 0)
            __builtin_amdgcn_global_load_lds(a.lse2 + so, (lds_void_t*)(st + 2 * T::BYTES), 4, 0, 0);
        if (wave == 1)
            __builtin_amdgcn_global_load_lds(a.dd + so, (lds_void_t*)(st + 2 * T::BYTES + BQ * 4), 4, 0, 0);
    };
    auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

    // The tile is two 32-query blocks. Per block: S = Q K^T and dP = dO V^T
    // (16 MFMAs), then P and dS (VALU), then dV^T += dO^T P and dK^T += Q^T dS
    // (16 MFMAs). With one wave per SIMD nothing hides latency but the wave's
    // own instruction order, so the tile is scheduled by hand: operand reads
    // run PF MFMAs ahead, and the softmax of one block is cut into slices
    // placed between the MFMAs of the next phase:
    //   S/dP(0); S/dP(1) + softmax(0); dV/dK(0) + softmax(1); dV/dK(1).
    // sched_barrier(0) fences keep the compiler from regrouping the stream.
    constexpr int PF = 3;                // prefetch distance, in MFMA pairs
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    struct Soft {                        // softmax state of one 32-query block
        f32x16 s, dp;
        float p[16], ds[16];
        bf16x8 pb[2], sb[2];
    };
    // Softmax slice k (0..5) of block mb: slices 0-3 handle element groups
    // g4 = k (4 elements each), slices 4-5 pack half k-4 into bf16 operands.
    auto soft_slice = [&](Soft& x, const float* Ls, const float* Ds, int mb, int thr, int k, auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        if (k < 4) {
            const int g4 = k;
            const int ql = mb * 32 + 8 * g4 + 4 * hi;   // tile-local query of element 4*g4
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int u = 4 * g4 + e;
                float sv = x.s[u];
                // Causal diagonal: key myk is invisible to queries before it;
                // thr is the key minus the element-0 query (very negative off
                // the diagonal).
                if constexpr (MASKED) sv = (thr > 8 * g4 + e) ? -INFINITY : sv;
                x.p[u] = exp2_fast(__builtin_fmaf(sv, c2, -l4[e]));
                x.ds[u] = x.p[u] * x.dp[u];   // dP accumulator started at -D
            }
        } else {
            const int half = k - 4;
            u32x4 wp, wd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wp[e] = pack_bf16x2(x.p[half * 8 + 2 * e], x.p[half * 8 + 2 * e + 1]);
                wd[e] = pack_bf16x2(x.ds[half * 8 + 2 * e], x.ds[half * 8 + 2 * e + 1]);
            }
            x.pb[half] = as_bf16x8(wp);
            x.sb[half] = as_bf16x8(wd);
        }
    };

    auto tile = [&](int s, int t, auto masked_c) {
        static_assert(MB == 2, "the schedule below is written for two 32-query blocks");
        constexpr bool masked = decltype(masked_c)::value;
        const int q0 = qstart + t * BQ;
        const unsigned char* Qs = stage_ptr(s);
        const unsigned char* Gs = Qs + T::BYTES;
        const float* Ls = reinterpret_cast<const float*>(Qs + 2 * T::BYTES);
        const float* Ds = Ls + BQ;
        const int thr[2] = {masked ? myk - (q0 + 4 * hi) : -(1 << 30), masked ? myk - (q0 + 32 + 4 * hi) : -(1 << 30)};
        Soft x[2];

        // Phase S/dP: step i in 0..2*DC-1 covers block i/DC, d chunk i%DC.
        bf16x8 ra[2 * DC], rb[2 * DC];
        auto row_load = [&](int i) {
            const int off = (rowb ^ ((i % DC) << 5)) + (i / DC) * 32 * RB;
            ra[i] = T::read_row(Qs, off);
            rb[i] = T::read_row(Gs, off);
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) row_load(i);
        fence();
#pragma unroll
        for (int i = 0; i < 2 * DC; ++i) {
            Soft& y = x[i / DC];
            const int cc = i % DC;
            if (cc == 0) {
                // dP - D: the accumulator starts at -D of its 16 query rows
                // (element u is query 8*(u/4) + 4*hi + u%4 of the block).
                y.s = f32x16{};
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + (i / DC) * 32 + 8 * g4 + 4 * hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) y.dp[4 * g4 + e] = d4[e];
                }
            }
            y.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i], kf[cc], y.s, 0, 0, 0);
            y.dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[i], vf[cc], y.dp, 0, 0, 0);
            if (i + PF < 2 * DC) row_load(i + PF);
            // Block 0's softmax runs under block 1's S/dP MFMAs.
            // (six slices spread over the DC steps of block 1)
            if (i >= DC) {
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    if (k * DC / 6 == i - DC) soft_slice(x[0], Ls, Ds, 0, thr[0], k, masked_c);
            }
            fence();
        }

        // Phase dV/dK: step j in 0..2*2*DB-1 covers block j/(2DB), d block
        // (j/2)%DB, 16-query half j%2.
        constexpr int NJ = 2 * 2 * DB;
        bf16x8 ta[NJ], tb[NJ];
        auto tr_load = [&](int j) {
            const int mb = j / (2 * DB), db = (j / 2) % DB, half = j % 2;
            const int qc = mb * 2 + half;
            const int o0 = (trb0 ^ (db << 6)) + qc * 16 * RB, o1 = (trb1 ^ (db << 6)) + qc * 16 * RB;
            ta[j] = T::read_tr(Gs, o0, o1);
            tb[j] = T::read_tr(Qs, o0, o1);
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) tr_load(j);
        fence();
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int mb = j / (2 * DB), db = (j / 2) % DB, half = j % 2;
            dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[j], x[mb].pb[half], dvacc[db], 0, 0, 0);
            dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[j], x[mb].sb[half], dkacc[db], 0, 0, 0);
            if (j + PF < NJ) tr_load(j + PF);
            // Block 1's softmax runs under block 0's dV/dK MFMAs.
            // (six slices spread over the 2*DB steps of block 0)
            if (mb == 0) {
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    if (k * (2 * DB) / 6 == j) soft_slice(x[1], Ls, Ds, 1, thr[1], k, masked_c);
            }
            fence();
        }
    };

    // Causal: only the first BK / BQ tiles (queries k0 .. k0+BK-1) straddle the
    // diagonal of this workgroup's keys; they run the masked variant, the
    // rest the variant without mask arithmetic.
    // With grouped-query attention the GS query heads of this workgroup are
    // processed one after the other, all accumulating into the same dK, dV;
    // the staged tiles run through them as one sequence n = g * ntiles + t.
    const int t_split = CAUSAL ? min(ntiles, BK / BQ) : 0;
    auto load_next = [&](int g, int t, int n) {
        int gn = g, tn = t + 1;
        if (tn == ntiles) {
            gn = g + 1;
            tn = 0;
        }
        if (gn < GS) dma(gn, tn, (n + 1) & 1);
    };
    dma(0, 0, 0);
    wait_dma();
    __syncthreads();
    if constexpr (!GQA) {
        for (int t = 0; t < t_split; ++t) {
            if (t + 1 < ntiles) dma(0, t + 1, (t + 1) & 1);
            // Tiles whose last query precedes this wave's first key are empty.
            if (qstart + t * BQ + BQ - 1 >= kw) tile(t & 1, t, std::true_type{});
            wait_dma();
            __syncthreads();
        }
        for (int t = t_split; t < ntiles; ++t) {
            if (t + 1 < ntiles) dma(0, t + 1, (t + 1) & 1);
            tile(t & 1, t, std::false_type{});
            wait_dma();
            __syncthreads();
        }
    } else {
        for (int g = 0; g < GS; ++g) {
            const int n0 = g * ntiles;
            for (int t = 0; t < t_split; ++t) {
                load_next(g, t, n0 + t);
                if (qstart + t * BQ + BQ - 1 >= kw) tile((n0 + t) & 1, t, std::true_type{});
                wait_dma();
                __syncthreads();
            }
            for (int t = t_split; t < ntiles; ++t) {
                load_next(g, t, n0 + t);
                tile((n0 + t) & 1, t, std::false_type{});
                wait_dma();
                __syncthreads();
            }
        }
    }

    if (GQA && S > 1) {
        // Partial sums of this part of the head group: fp32, dK unscaled.
        if (myk < N) {
            const size_t elems = (size_t)B * N * Hkv * D;
            float* pk = a.part + (size_t)(2 * sp) * elems + kvbase + (size_t)myk * rskv;
            float* pv = pk + elems;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + 8 * g + 4 * hi;
                    st16f(pk + d0, f32x4{dkacc[db][4 * g], dkacc[db][4 * g + 1], dkacc[db][4 * g + 2],
                                         dkacc[db][4 * g + 3]});
                    st16f(pv + d0, f32x4{dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2],
                                         dvacc[db][4 * g + 3]});
                }
        }
        return;
    }
    // dK, then dV, leave through LDS (this wave's part of the tile stages,
    // idle since the last barrier) as whole 16-byte chunks of key rows.
    static_assert(NW * 32 * RB <= 2 * STAGE, "dK/dV staging fits the tile stages");
    unsigned char* sw = smem + wave * 32 * RB;
    stage_rows<D>(sw, dkacc, a.scale, l32, hi);
    store_rows<D>(static_cast<__bf16*>(a.dk) + kvbase, rskv, sw, kw, N, lane);
    stage_rows<D>(sw, dvacc, 1.0f, l32, hi);
    store_rows<D>(static_cast<__bf16*>(a.dv) + kvbase, rskv, sw, kw, N, lane);
}

// ---------------------------------------------------------------------------
// dK, dV for d = 128: one workgroup of 8 waves per 128 keys, looping over
// query tiles of 64 rows staged in LDS by direct loads. At d = 128 the four
// products of a wave that owns 32 keys need more than 256 VGPRs (K, V, dK, dV
// alone take 192), which would leave one wave per SIMD. Instead waves w and
// w + 4 share the 32 keys k0 + 32 (w % 4) .. +31 and run on the same SIMD
// with complementary work:
//
//   P wave  (w < 4):  S = Q K^T, P = exp2(S c2 - LSE2) (K rows in VGPRs),
//                     dV^T += dO^T P; P goes to LDS for the partner as the
//                     bf16 pairs the dV product uses.
//   dS wave (w >= 4): dP - D = dO V^T - D (V rows in VGPRs; the accumulator
//                     starts at -D); one tile later, with the partner's P,
//                     dS = P o (dP - D) and dK^T += Q^T dS.
//
// Either wave holds one set of key rows and one 32 x d accumulator, so two
// waves fit a SIMD's registers, and while one wave is in its exponential or
// product phase the other keeps the matrix core busy. The dS wave lags its
// partner by one tile, so Q tiles are triple-buffered (the dS wave still
// reads tile n - 1 while tile n + 1 loads) and everything else double-
// buffered; one barrier per tile orders every LDS hand-over.
//
// In the 32x32 accumulators of S and dP each lane holds one key column
// (lane % 32) and 16 query rows, which is exactly the B operand layout of
// dV^T += dO^T P and dK^T += Q^T dS; their A operands come from transposing
// reads of the dO and Q tiles.
template <int D, bool CAUSAL, bool GQA>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdArgs a) {
    using T = LdsTile<D>;
    constexpr int NW = 8;
    constexpr int BK = 128;              // keys per workgroup
    constexpr int BQ = T::ROWS;          // queries per tile
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int MB = BQ / 32;          // 32-query blocks per tile
    constexpr int RB = T::RB;
    static_assert(MB == 2, "the schedule below is written for two 32-query blocks");
    constexpr int SST = 2 * BQ * 4;                    // statistics stage: LSE2[BQ], -D[BQ]
    constexpr int PXG = MB * 2 * 1024;                 // P (bf16) of one key group: per block, 2 rows of 1 KB
    constexpr int PXB = 4 * PXG;                       // P exchange buffer (4 key groups)
    constexpr int QOFF = 0;                            // Q tiles, 3 stages
    constexpr int GOFF = 3 * T::BYTES;                 // dO tiles, 2 stages
    constexpr int SOFF = 5 * T::BYTES;                 // statistics, 2 stages
    constexpr int POFF = SOFF + 2 * SST;               // P exchange, 2 buffers
    constexpr int LDS_BYTES = POFF + 2 * PXB;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];
    lds_poison(smem, sizeof(smem));

    const int B = a.B, H = a.H, N = a.N;
    const int npad = (N + 63) & ~63;
    const int Hkv = GQA ? a.Hkv : H;
    const int G = GQA ? H / Hkv : 1;     // query heads sharing this K/V head
    // Grouped-query split: the G heads run as S workgroups of GS heads each,
    // which write fp32 partial sums (reduced by bwd_dkdv_reduce_kernel).
    const int S = GQA ? a.gsplit : 1;
    const int GS = G / S;
    const int nk = (N + BK - 1) / BK;
    int unit, kb;                        // causal: low key blocks see the most query tiles, so go first
    work_item(blockIdx.x, nk, B * Hkv * S, CAUSAL, unit, kb);
    const int bhk = GQA ? unit / S : unit;
    const int sp = GQA ? unit - bhk * S : 0;   // part of the head group
    const int b = bhk / Hkv, hk = bhk - b * Hkv;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int kg = wave & 3;             // key group
    const bool pwave = wave < 4;

    const size_t rs = (size_t)H * D;                  // Q / dO row stride
    const size_t rskv = (size_t)Hkv * D;              // K / V / dK / dV row stride
    const size_t kvbase = ((size_t)b * N * Hkv + hk) * D;
    // Query head g of this workgroup's part is h = hk * G + sp * GS + g: its
    // Q / dO start D elements after head g - 1's, its statistics npad floats after.
    const size_t qbase = ((size_t)b * N * H + (size_t)hk * G + (size_t)sp * GS) * D;
    const __bf16* Qg0 = static_cast<const __bf16*>(a.q) + qbase;
    const __bf16* dOg0 = static_cast<const __bf16*>(a.dO) + qbase;
    const size_t stat0 = ((size_t)b * H + (size_t)hk * G + (size_t)sp * GS) * npad;

    const int k0 = kb * BK;
    const int kw = k0 + kg * 32;         // first key of this wave
    const int myk = kw + l32;            // key column owned by this lane

    // Key rows as B operands (lane holds row myk, d chunk c*16 + hi*8 .. +8):
    // K for the P wave (negative scale folded into its sign), V for the dS wave.
    bf16x8 rf[DC];
    {
        const __bf16* Rg = static_cast<const __bf16*>(pwave ? a.k : a.v) + kvbase;
        const uint32_t sgn = pwave ? a.qsign : 0u;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (myk < N) x = ld16(Rg + (size_t)myk * rskv + c * 16 + hi * 8);
            x ^= sgn;
            rf[c] = as_bf16x8(x);
        }
    }

    f32x16 acc[DB];                      // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

    const int qstart = CAUSAL ? k0 : 0;  // k0 is a multiple of BQ
    const int ntiles = (N - qstart + BQ - 1) / BQ;
    const float c2 = a.c2;
    const int rowb = T::rowbase(lane);
    const int trb0 = T::trbase(lane, 0);
    const int trb1 = T::trbase(lane, 1);

    auto qtile = [&](int s) { return smem + QOFF + s * T::BYTES; };
    auto gtile = [&](int s) { return smem + GOFF + s * T::BYTES; };
    auto stats = [&](int s) { return reinterpret_cast<float*>(smem + SOFF + s * SST); };
    auto pxch = [&](int s) { return reinterpret_cast<uint32_t*>(smem + POFF + s * PXB + kg * PXG); };

    // Only the P waves load tiles: a direct load stalls the issuing wave until
    // the memory pipeline accepts it, and the P waves have slack at the
    // barrier while the dS waves are the critical path.
    constexpr int NL = 4;                // loading waves
    unsigned toff[T::NINST / NL];
    T::template offsets<NL>(toff, rs, kg, lane);
    // Tile t of group head g: Q into Q stage qs, dO and statistics into stage gs.
    // Query head 0 of the group part loads through a buffer resource over its rows.
    const uint32_t qspan = T::span(rs, N);
    auto dma = [&](int g, int t, int qs, int gs) {
        if (!pwave) return;
        const int q0 = qstart + t * BQ;
        if (GQA && g > 0) {
            T::template load<NL>(qtile(qs), Qg0 + (size_t)g * D, rs, q0, N, kg, lane, toff);
            T::template load<NL>(gtile(gs), dOg0 + (size_t)g * D, rs, q0, N, kg, lane, toff);
        } else {
            T::template load_buf<NL>(qtile(qs), Qg0, qspan, rs, q0, N, kg, lane, toff);
            T::template load_buf<NL>(gtile(gs), dOg0, qspan, rs, q0, N, kg, lane, toff);
        }
        // q0 + 63 < npad: the padded statistics need no clamp.
        const size_t so = stat0 + (size_t)g * npad + q0 + lane;
        if (kg == 0) __builtin_amdgcn_global_load_lds(a.lse2 + so, (lds_void_t*)stats(gs), 4, 0, 0);
        if (kg == 1) __builtin_amdgcn_global_load_lds(a.dd + so, (lds_void_t*)(stats(gs) + BQ), 4, 0, 0);
    };
    auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

    // Operand reads run PF MFMAs ahead of their use; sched_barrier(0) fences
    // keep the compiler from regrouping the hand-placed stream.
    constexpr int PF = 3;
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // MFMAs of the dV (or dK) phase: step j covers block j / (2 DB), 16-query
    // half (j / DB) % 2 and d block j % DB, so consecutive products update
    // different accumulators (each accumulator still sums in the same order).
    constexpr int NJ = 2 * 2 * DB;
    auto tr_off = [&](int j, int& o0, int& o1) {
        const int mb = j / (2 * DB), half = (j / DB) % 2, db = j % DB;
        const int qc = mb * 2 + half;
        o0 = (trb0 ^ (db << 6)) + qc * 16 * RB;
        o1 = (trb1 ^ (db << 6)) + qc * 16 * RB;
    };
    auto row_off = [&](int i) { return (rowb ^ ((i % DC) << 5)) + (i / DC) * 32 * RB; };

    // ---- P wave: one tile -------------------------------------------------
    // S = Q K^T (16 MFMAs), then dV^T += dO^T P (16 MFMAs). The softmax of
    // block 0 runs in 8 parts under block 1's S MFMAs, block 1's under
    // block 0's dV MFMAs. Part k computes elements 2k, 2k+1; odd parts also
    // store the finished group of four to LDS and pack it to bf16.
    auto p_tile = [&](int qs, int gs, int t, auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int q0 = qstart + t * BQ;
        const unsigned char* Qs = qtile(qs);
        const unsigned char* Gs = gtile(gs);
        const float* Ls = stats(gs);
        uint32_t* Px = pxch(gs);
        // Causal diagonal: key myk is invisible to queries before it; thr is
        // the key minus the element-0 query of the block.
        const int thr[2] = {MASKED ? myk - (q0 + 4 * hi) : 0, MASKED ? myk - (q0 + 32 + 4 * hi) : 0};
        f32x16 s[2];
        f32x4 l4[2][4];
        u32x4 pk[2][2];
        auto soft = [&](int mb, int k) {
#pragma unroll
            for (int e = 2 * k; e < 2 * k + 2; ++e) {
                float sv = s[mb][e];
                if constexpr (MASKED) sv = (thr[mb] > 8 * (e >> 2) + (e & 3)) ? -INFINITY : sv;
                s[mb][e] = exp2_fast(__builtin_fmaf(sv, c2, -l4[mb][e >> 2][e & 3]));
            }
            if (k & 1) {
                const int g4 = k >> 1;
                pk[mb][g4 >> 1][2 * (g4 & 1)] = pack_bf16x2(s[mb][4 * g4], s[mb][4 * g4 + 1]);
                pk[mb][g4 >> 1][2 * (g4 & 1) + 1] = pack_bf16x2(s[mb][4 * g4 + 2], s[mb][4 * g4 + 3]);
                // P goes to the dS wave as the bf16 pairs dV uses: 16 bytes
                // per lane once a group of eight is packed.
                if (g4 & 1) *reinterpret_cast<u32x4*>(Px + (mb * 2 + (g4 >> 1)) * 256 + lane * 4) = pk[mb][g4 >> 1];
            }
        };
        bf16x8 ra[2 * DC];
        auto row_load = [&](int i) { ra[i] = T::read_row(Qs, row_off(i)); };
#pragma unroll
        for (int i = 0; i < PF; ++i) row_load(i);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) l4[0][g4] = *reinterpret_cast<const f32x4*>(Ls + 8 * g4 + 4 * hi);
        fence();
#pragma unroll
        for (int i = 0; i < 2 * DC; ++i) {
            const int mb = i / DC;
            if (i % DC == 0) s[mb] = f32x16{};
            s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i], rf[i % DC], s[mb], 0, 0, 0);
            if (i + PF < 2 * DC) row_load(i + PF);
            if (i == DC - 1) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    l4[1][g4] = *reinterpret_cast<const f32x4*>(Ls + 32 + 8 * g4 + 4 * hi);
            }
            if (i >= DC) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (k * DC / 8 == i - DC) soft(0, k);
            }
            fence();
        }
        bf16x8 ta[NJ];
        auto tr_load = [&](int j) {
            int o0, o1;
            tr_off(j, o0, o1);
            ta[j] = T::read_tr(Gs, o0, o1);
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) tr_load(j);
        fence();
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int mb = j / (2 * DB), half = (j / DB) % 2, db = j % DB;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[j], as_bf16x8(pk[mb][half]), acc[db], 0, 0, 0);
            if (j + PF < NJ) tr_load(j + PF);
            if (mb == 0) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (k * (2 * DB) / 8 == j) soft(1, k);
            }
            fence();
        }
    };

    // ---- dS wave: one step -------------------------------------------------
    // prev: finish the previous tile (its P in exchange buffer pgs, its Q in
    // stage qsp): dS = P o (dP - D), then dK^T += Q^T dS (16 MFMAs).
    // cur: dP - D of the current tile (dO stage gs; 16 MFMAs), kept in dp for
    // the next step. Block 0's dS is done before block 0's accumulator is
    // re-seeded; block 1's runs under block 0's dP MFMAs.
    f32x16 dp[2];
    auto ds_step = [&](int gs, int qsp, int pgs, bool prev, bool cur) {
        const unsigned char* Gs = gtile(gs);
        const float* Ds = stats(gs) + BQ;
        const unsigned char* Qp = qtile(qsp);
        const uint32_t* Pp = pxch(pgs);
        u32x4 pr[2][2];
        u32x4 sk[2][2];
        auto ds_part = [&](int mb, int k) {
            // Elements 2k, 2k+1: one packed bf16 pair of P (low half first).
            const uint32_t w = pr[mb][k >> 2][k & 3];
            const float v0 = __uint_as_float(w << 16) * dp[mb][2 * k];
            const float v1 = __uint_as_float(w & 0xffff0000u) * dp[mb][2 * k + 1];
            sk[mb][k >> 2][k & 3] = pack_bf16x2(v0, v1);
        };
        bf16x8 rb[2 * DC];
        auto row_load = [&](int i) { rb[i] = T::read_row(Gs, row_off(i)); };
        if (prev) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    pr[mb][h2] = *reinterpret_cast<const u32x4*>(Pp + (mb * 2 + h2) * 256 + lane * 4);
        }
        if (cur) {
#pragma unroll
            for (int i = 0; i < PF; ++i) row_load(i);
        }
        fence();
        if (prev) {
#pragma unroll
            for (int k = 0; k < 8; ++k) ds_part(0, k);
        }
        fence();
        if (cur) {
#pragma unroll
            for (int i = 0; i < 2 * DC; ++i) {
                const int mb = i / DC;
                if (i % DC == 0) {
                    // The accumulator starts at -D of its 16 query rows
                    // (element u is query 8*(u/4) + 4*hi + u%4 of the block).
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + mb * 32 + 8 * g4 + 4 * hi);
#pragma unroll
                        for (int e = 0; e < 4; ++e) dp[mb][4 * g4 + e] = d4[e];
                    }
                }
                dp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[i], rf[i % DC], dp[mb], 0, 0, 0);
                if (i + PF < 2 * DC) row_load(i + PF);
                if (prev && i < DC) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (k * DC / 8 == i) ds_part(1, k);
                }
                fence();
            }
        } else if (prev) {
#pragma unroll
            for (int k = 0; k < 8; ++k) ds_part(1, k);
        }
        if (prev) {
            bf16x8 tb[NJ];
            auto tr_load = [&](int j) {
                int o0, o1;
                tr_off(j, o0, o1);
                tb[j] = T::read_tr(Qp, o0, o1);
            };
#pragma unroll
            for (int j = 0; j < PF; ++j) tr_load(j);
            fence();
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int mb = j / (2 * DB), half = (j / DB) % 2, db = j % DB;
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[j], as_bf16x8(sk[mb][half]), acc[db], 0, 0, 0);
                if (j + PF < NJ) tr_load(j + PF);
                fence();
            }
        }
    };

    // Tiles run as one sequence n over (group head g, tile t). Causal: only
    // the first BK / BQ tiles of a head (queries k0 .. k0+BK-1) straddle the
    // diagonal; they run the masked variant. A tile whose last query precedes
    // a wave's first key is empty for that key group and skipped by both of
    // its waves. Both roles pass the same barriers, one per tile.
    const int t_split = CAUSAL ? min(ntiles, BK / BQ) : 0;
    auto nonempty = [&](int t) { return !CAUSAL || qstart + t * BQ + BQ - 1 >= kw; };
    auto dma_next = [&](int g, int t, int qs, int gs) {
        int gn = g, tn = t + 1;
        if (tn == ntiles) {
            gn = g + 1;
            tn = 0;
        }
        if (gn < GS) dma(gn, tn, qs == 2 ? 0 : qs + 1, gs ^ 1);
    };
    dma(0, 0, 0, 0);
    wait_dma();
    __syncthreads();
    int qs = 0, n = 0;
    if (pwave) {
        auto step = [&](int g, int t, auto masked_c) {
            const int gs = n & 1;
            dma_next(g, t, qs, gs);
            if (nonempty(t)) p_tile(qs, gs, t, masked_c);
            wait_dma();
            __syncthreads();
            qs = qs == 2 ? 0 : qs + 1;
            ++n;
        };
        for (int g = 0; g < GS; ++g) {
            for (int t = 0; t < t_split; ++t) step(g, t, std::true_type{});
            for (int t = t_split; t < ntiles; ++t) step(g, t, std::false_type{});
        }
    } else {
        bool prev = false;
        for (int g = 0; g < GS; ++g) {
            for (int t = 0; t < ntiles; ++t) {
                const int gs = n & 1;
                dma_next(g, t, qs, gs);
                const bool cur = nonempty(t);
                ds_step(gs, qs == 0 ? 2 : qs - 1, gs ^ 1, prev, cur);
                prev = cur;
                wait_dma();
                __syncthreads();
                qs = qs == 2 ? 0 : qs + 1;
                ++n;
            }
        }
        ds_step(0, qs == 0 ? 2 : qs - 1, (n - 1) & 1, prev, false);
    }

    if (GQA && S > 1) {
        // Partial sums of this part of the head group: fp32, dK unscaled.
        if (myk < N) {
            const size_t elems = (size_t)B * N * Hkv * D;
            float* prow = a.part + (size_t)(2 * sp + (pwave ? 1 : 0)) * elems + kvbase + (size_t)myk * rskv;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    st16f(prow + db * 32 + 8 * g + 4 * hi,
                          f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]});
        }
        return;
    }
    // dV (P wave) or dK (dS wave) leaves through LDS as whole 16-byte chunks
    // of key rows, once every wave is past its last LDS read (the dS wave's
    // final step above).
    __syncthreads();
    static_assert(NW * 32 * RB <= LDS_BYTES, "dK/dV staging fits the LDS");
    unsigned char* sw = smem + wave * 32 * RB;
    stage_rows<D>(sw, acc, pwave ? 1.0f : a.scale, l32, hi);
    store_rows<D>(static_cast<__bf16*>(pwave ? a.dv : a.dk) + kvbase, rskv, sw, kw, N, lane);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup of NW = 8 or 4 waves (two per SIMD) per 32*NW queries
// (32 per wave, Q and dO rows in VGPRs), looping over key tiles of 64 rows
// staged in LDS by direct loads, double-buffered. S^T = K Q^T and dP^T = V dO^T use row reads of the K and V
// tiles; dQ^T += K^T dS^T takes its A operand from transposing reads of the
// same K tile. The accumulators hold one query per lane, as in the forward.
//
// PREP: the kernel also does bwd_pre's work for its own queries. Each lane
// already holds half of its query's dO row; it loads the same half of the O
// row and forms -D and LSE * log2(e) in registers, and writes both into the
// workspace for the dK/dV kernel, which then runs after this one. The dot
// product is summed in exactly bwd_pre's order (8 products per 16-byte
// chunk, then the chunks pairwise as its butterfly over 16 threads pairs
// them), so the statistics, and with them dQ, dK and dV, are bitwise those of
// the separate preprocess.
template <int D, bool CAUSAL, int NW, bool PREP>
__global__ __launch_bounds__(NW * 64, D == 64 ? 3 : 8 / NW) void bwd_dq_kernel(BwdArgs a) {
    using T = LdsTile<D>;
    constexpr int BM = NW * 32;          // queries per workgroup
    constexpr int BN = T::ROWS;          // keys per tile
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int KB = BN / 32;
    constexpr int RB = T::RB;

    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * T::BYTES];   // Kbuf[2], Vbuf[2]
    lds_poison(smem, sizeof(smem));

    const int B = a.B, H = a.H, N = a.N;
    const int npad = (N + 63) & ~63;
    const int nq = (N + BM - 1) / BM;
    int bh, qb;
    work_item(blockIdx.x, nq, B * H, CAUSAL, bh, qb);
    if (CAUSAL) qb = nq - 1 - qb;        // longest rows first
    const int b = bh / H, h = bh - b * H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;                  // Q / dO / dQ row stride
    const size_t base = ((size_t)b * N * H + h) * D;
    const int hk = h / (H / a.Hkv);                   // K / V head of this query head
    const size_t rskv = (size_t)a.Hkv * D;
    const size_t kvbase = ((size_t)b * N * a.Hkv + hk) * D;
    const __bf16* Qg = static_cast<const __bf16*>(a.q) + base;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + kvbase;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + kvbase;
    const __bf16* dOg = static_cast<const __bf16*>(a.dO) + base;

    const int q0 = qb * BM;
    const int qw = q0 + wave * 32;
    const int myq = qw + l32;

    bf16x8 qf[DC], gf[DC];
    // PREP: this lane's half of its O row. Loaded for every lane (rows past
    // the end read row N - 1, and their statistics are discarded below), so
    // that no wait for these loads is needed before the first tile's loads.
    u32x4 orow[PREP ? DC : 1];
    if constexpr (PREP) {
        const __bf16* Or = static_cast<const __bf16*>(a.o) + base + (size_t)min(myq, N - 1) * rs + hi * 8;
#pragma unroll
        for (int c = 0; c < DC; ++c) orow[c] = ld16(Or + c * 16);
    }
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
    float lse2 = 0.f, ndd = 0.f;         // LSE * log2(e) and -D of this lane's query
    float lse_in = 0.f;
    if constexpr (PREP) {
        lse_in = a.lse[(size_t)bh * N + min(myq, N - 1)];   // discarded past the end, as the O row
    } else {
        lse2 = (myq < N) ? a.lse2[(size_t)bh * npad + myq] : 0.f;
        ndd = (myq < N) ? a.dd[(size_t)bh * npad + myq] : 0.f;
    }
    // PREP, once the first K/V tile's loads are in flight (so that the wait
    // for the O rows does not delay them): -D and LSE * log2(e), written to
    // the workspace by the lanes of the lower half.
    auto preprocess = [&] {
        float part[DC];                  // dO . O over each 16-byte chunk of the row
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const u32x4 ov = orow[c];
            const u32x4 gv = as_u32x4(gf[c]);
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc += __uint_as_float(ov[w] << 16) * __uint_as_float(gv[w] << 16);
                acc += __uint_as_float(ov[w] & 0xffff0000u) * __uint_as_float(gv[w] & 0xffff0000u);
            }
            part[c] = acc;
        }
        // Chunk j = 2c + hi of the row; bwd_pre's butterfly adds chunks j ^ 8,
        // then j ^ 4, j ^ 2 and j ^ 1: c ^ (DC/2) ... c ^ 1 here, then the halves.
#pragma unroll
        for (int w = DC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int c = 0; c < w; ++c) part[c] = part[c] + part[c + w];
        const float dsum = sum_halves(part[0]);
        lse2 = (myq < N) ? lse_in * kLog2e : 0.f;
        ndd = (myq < N) ? -dsum : 0.f;
        if (hi == 0 && myq < npad) {
            const size_t i = (size_t)bh * npad + myq;
            a.dd[i] = ndd;
            a.lse2[i] = (myq < N) ? lse2 : INFINITY;
        }
    };

    f32x16 dqacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dqacc[i] = f32x16{};

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;
    const float c2 = a.c2;
    const int rowb = T::rowbase(lane);
    const int trb0 = T::trbase(lane, 0);
    const int trb1 = T::trbase(lane, 1);

    auto kbuf = [&](int s) { return smem + s * T::BYTES; };
    auto vbuf = [&](int s) { return smem + (2 + s) * T::BYTES; };
    unsigned toff[T::NINST / NW];
    T::template offsets<NW>(toff, rskv, wave, lane);
    const uint32_t kvspan = T::span(rskv, N);
    auto dma = [&](int t, int s) {
        T::template load_buf<NW>(kbuf(s), Kg, kvspan, rskv, t * BN, N, wave, lane, toff);
        T::template load_buf<NW>(vbuf(s), Vg, kvspan, rskv, t * BN, N, wave, lane, toff);
    };
    auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

    // Per tile: for each 32-key block, S^T and dP^T (16 MFMAs) then dS (VALU);
    // then dQ^T += K^T dS^T (16 MFMAs). Operand reads are issued PF MFMAs
    // ahead of their use and fenced so the compiler keeps that order.
    constexpr int PF = 4;
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto tile = [&](int t, auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int j0 = t * BN;
        const unsigned char* Ks = kbuf(t & 1);
        const unsigned char* Vs = vbuf(t & 1);
        bf16x8 sb[BN / 16];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x16 s = f32x16{}, dp = f32x16{};
            bf16x8 ra[DC], rb[DC];
            auto row_load = [&](int cc) {
                const int off = (rowb ^ (cc << 5)) + kb * 32 * RB;
                ra[cc] = T::read_row(Ks, off);
                rb[cc] = T::read_row(Vs, off);
            };
#pragma unroll
            for (int cc = 0; cc < PF; ++cc) row_load(cc);
            fence();
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[cc], qf[cc], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[cc], gf[cc], dp, 0, 0, 0);
                if (cc + PF < DC) row_load(cc + PF);
                fence();
            }
            if constexpr (MASKED) {
                // Keys past the end, and under the causal mask keys after the
                // query. Key of element u is j0 + kb*32 + 4*hi + 8*(u/4) + u%4.
                const int thr = (CAUSAL ? min(N - 1, myq) : N - 1) - (j0 + kb * 32 + 4 * hi);
#pragma unroll
                for (int u = 0; u < 16; ++u) s[u] = (8 * (u >> 2) + (u & 3) > thr) ? -INFINITY : s[u];
            }
            float ds[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) ds[u] = exp2_fast(__builtin_fmaf(s[u], c2, -lse2)) * (dp[u] + ndd);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(ds[half * 8 + 2 * e], ds[half * 8 + 2 * e + 1]);
                sb[kb * 2 + half] = as_bf16x8(w);
            }
            fence();
        }
        constexpr int NJ = DB * (BN / 16);
        bf16x8 ka[NJ];
        auto tr_load = [&](int j) {
            const int db = j / (BN / 16), kc = j % (BN / 16);
            ka[j] = T::read_tr(Ks, (trb0 ^ (db << 6)) + kc * 16 * RB, (trb1 ^ (db << 6)) + kc * 16 * RB);
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) tr_load(j);
        fence();
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int db = j / (BN / 16), kc = j % (BN / 16);
            dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], sb[kc], dqacc[db], 0, 0, 0);
            if (j + PF < NJ) tr_load(j + PF);
            fence();
        }
    };

    // Tiles before t_split need no mask for any wave of the workgroup (they
    // end before the first query and before N); the rest run the masked
    // variant. The split keeps mask arithmetic out of the main loop.
    const int t_split = min(CAUSAL ? q0 / BN : ntiles, (N % BN) ? ntiles - 1 : ntiles);
    dma(0, 0);
    if constexpr (PREP) preprocess();
    wait_dma();
    __syncthreads();
    for (int t = 0; t < t_split; ++t) {
        if (t + 1 < ntiles) dma(t + 1, (t + 1) & 1);
        tile(t, std::false_type{});
        wait_dma();
        __syncthreads();
    }
    for (int t = t_split; t < ntiles; ++t) {
        if (t + 1 < ntiles) dma(t + 1, (t + 1) & 1);
        if (!CAUSAL || t * BN <= qw + 31) tile(t, std::true_type{});
        wait_dma();
        __syncthreads();
    }

    // dQ leaves through LDS (this wave's part of the K/V buffers, idle since
    // the last barrier) as whole 16-byte chunks of rows.
    static_assert(NW * 32 * RB <= 4 * T::BYTES, "dQ staging fits the K/V buffers");
    unsigned char* sw = smem + wave * 32 * RB;
    stage_rows<D>(sw, dqacc, a.scale, l32, hi);
    store_rows<D>(static_cast<__bf16*>(a.dq) + base, rs, sw, qw, N, lane);
}

// Split grouped-query dK/dV: sums the gsplit fp32 partials of each element in
// part order (so the result is deterministic), multiplies dK by the scale and
// rounds both to bf16. One thread per 8 consecutive elements of dK or dV.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdArgs a) {
    const size_t elems = (size_t)a.B * a.N * a.Hkv * D;
    const size_t n8 = elems / 8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= 2 * n8) return;
    const int role = i >= n8;            // 0: dK, 1: dV
    const size_t e = (i - (size_t)role * n8) * 8;
    const float* p = a.part + (size_t)role * elems + e;
    f32x4 s0 = *reinterpret_cast<const f32x4*>(p);
    f32x4 s1 = *reinterpret_cast<const f32x4*>(p + 4);
    for (int sp = 1; sp < a.gsplit; ++sp) {
        p += 2 * elems;
        s0 += *reinterpret_cast<const f32x4*>(p);
        s1 += *reinterpret_cast<const f32x4*>(p + 4);
    }
    const float sc = role ? 1.0f : a.scale;
    u32x4 w;
    w[0] = pack_bf16x2(s0[0] * sc, s0[1] * sc);
    w[1] = pack_bf16x2(s0[2] * sc, s0[3] * sc);
    w[2] = pack_bf16x2(s1[0] * sc, s1[1] * sc);
    w[3] = pack_bf16x2(s1[2] * sc, s1[3] * sc);
    st16(static_cast<__bf16*>(role ? a.dv : a.dk) + e, w);
}

template <int D>
static hipError_t launch_prep(const BwdArgs& a, hipStream_t stream) {
    const long long blocks = (long long)a.B * a.H * (((a.N + 63) & ~63) / 64);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
    const int S = a.Hkv == a.H ? 1 : a.gsplit;
    const long long g = (long long)((a.N + 127) / 128) * a.B * a.Hkv * S;
    // d = 128: the 8-wave P / dS pair kernel (7-8% faster at 16k tokens).
    // d = 64: the 4-wave kernel, which already fits two workgroups per CU.
    if constexpr (D == 128) {
        if (a.Hkv == a.H)
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL, false>), dim3((unsigned)g), dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL, true>), dim3((unsigned)g), dim3(512), 0, stream, a);
    } else {
        if (a.Hkv == a.H)
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, false>), dim3((unsigned)g), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, true>), dim3((unsigned)g), dim3(256), 0, stream, a);
    }
    if (S > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long long threads = 2LL * a.B * a.N * a.Hkv * D / 8;
        hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool PREP>
static hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
    // 4-wave workgroups (two per CU at d = 128, three at d = 64) for d = 64
    // and for d = 128 up to 2048 tokens, as in the forward (measured: 5-26%
    // faster there; 8 waves win for d = 128 from 4096 tokens on).
    if constexpr (D == 128) {
        if (a.N > 2048) {
            const long long g = (long long)((a.N + 255) / 256) * a.B * a.H;
            hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, 8, PREP>), dim3((unsigned)g), dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    const long long g = (long long)((a.N + 127) / 128) * a.B * a.H;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, 4, PREP>), dim3((unsigned)g), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, int d, hipStream_t stream) {
    return d == 128 ? launch_prep<128>(a, stream) : launch_prep<64>(a, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch_dkdv<128, true>(a, stream) : launch_dkdv<128, false>(a, stream);
    return causal ? launch_dkdv<64, true>(a, stream) : launch_dkdv<64, false>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, bool prep, hipStream_t stream) {
    if (prep) {
        if (d == 128) return causal ? launch_dq<128, true, true>(a, stream) : launch_dq<128, false, true>(a, stream);
        return causal ? launch_dq<64, true, true>(a, stream) : launch_dq<64, false, true>(a, stream);
    }
    if (d == 128) return causal ? launch_dq<128, true, false>(a, stream) : launch_dq<128, false, false>(a, stream);
    return causal ? launch_dq<64, true, false>(a, stream) : launch_dq<64, false, false>(a, stream);
}

}  // namespace fa
