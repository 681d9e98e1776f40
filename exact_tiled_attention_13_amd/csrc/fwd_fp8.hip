// fwd_fp8.hip -- FP8 (E4M3) forward of exact tiled attention for gfx950.
//
// The page "FlashAttention-T: Optimización GPU para LLMs Escalables" (section
// "Innovaciones técnicas frente a FlashAttention original") names 8-bit
// quantisation as a supported mode and gives no algorithm. Reading used here:
// Q, K and V arrive as OCP E4M3 values with fp32 per-tensor descales
// (real = value * descale); S = Q K^T runs on the FP8 matrix cores with fp32
// accumulation, the online softmax is the forward's (fp32, base 2, running
// max over 64-key tiles), and P = exp2(S c2 - m) <= 1 is rounded to E4M3 for
// the P V product while the row sum uses the unrounded P. O is written in
// bf16 and LSE in fp32.
//
// CDNA4 mapping (4 waves, 32 query rows each, 128 per workgroup):
//   S^T = K Q^T     v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3): A = 32 K rows
//                   from LDS, B = Q^T from VGPRs; lane (row, half h) supplies
//                   the 32 bytes d = 64 c + 32 h .. +31 of both operands.
//   O^T += V^T P^T  A = V^T rows (d) from LDS: V is passed transposed
//                   ([B, H, d, ldv], keys contiguous), because both operands
//                   of the FP8 MFMA must be contiguous along the contraction;
//                   B = P^T: lane (query, h) supplies keys 32 h .. 32 h + 31.
//                   The score accumulators hold, per lane, 16 keys of each
//                   32-key block (4h + {0..3} + 8g); after packing to E4M3,
//                   one v_permlane32_swap per group gives each lane half the
//                   32 keys of one block.
//   K and V^T tiles are double-buffered in LDS and fetched by direct-to-LDS
//   loads, with 16-byte chunks XOR-swizzled per row so that the operand reads
//   (16 rows at one chunk column per 16 lanes) are free of bank conflicts.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds8_void_t;

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // Both operands E4M3 (format selectors 0); no block scales.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four floats -> four E4M3 bytes (round to nearest even), element 0 in the low byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

}  // namespace

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_fp8_kernel(Fp8Args a) {
    constexpr int BM = NW * 32;           // query rows per workgroup
    constexpr int BN = 64;                // keys per tile
    constexpr int KRB = D;                // bytes per K row
    constexpr int KCH = KRB / 16;         // 16-byte chunks per K row
    constexpr int VRB = BN;               // bytes per V^T row (one row per d)
    constexpr int TILE = BN * D;          // bytes per K or V^T tile
    constexpr int NINST = TILE / 1024;    // 1 KB direct-to-LDS wave loads per tile
    constexpr int IPW = NINST / NW;
    constexpr int DC = D / 64;            // 64-byte d chunks (MFMA K steps of S)
    constexpr int DB = D / 32;            // 32-wide d blocks of O^T
    static_assert(D == 128, "the FP8 forward is written for d = 128");
    static_assert(IPW * NW == NINST, "tile loads must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILE];   // K[2], V^T[2]
    lds_poison(smem, sizeof(smem));

    const int B = a.B, H = a.H, N = a.N;
    const int nq = (N + BM - 1) / BM;
    int bh, qb;
    work_item(blockIdx.x, nq, B * H, CAUSAL, bh, qb);
    if (CAUSAL) qb = nq - 1 - qb;         // longest rows first
    const int b = bh / H, h = bh - b * H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;                       // Q / K / O row stride (elements)
    const size_t base = ((size_t)b * N * H + h) * D;       // (b, 0, h, 0)
    const unsigned char* Qg = static_cast<const unsigned char*>(a.q) + base;
    const unsigned char* Kg = static_cast<const unsigned char*>(a.k) + base;
    const unsigned char* Vg = static_cast<const unsigned char*>(a.vt) + ((size_t)b * H + h) * D * a.ldv;
    __bf16* Og = static_cast<__bf16*>(a.o) + base;

    const int q0 = qb * BM;
    const int qw = q0 + wave * 32;
    const int myq = qw + l32;

    // Q^T (B operand of the score MFMAs): bytes d = 64 c + 32 hi .. +31 of row myq.
    i32x8 qf[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        u32x4 lo = {0u, 0u, 0u, 0u}, up = {0u, 0u, 0u, 0u};
        if (myq < N) {
            lo = ld16(Qg + (size_t)myq * rs + 64 * c + 32 * hi);
            up = ld16(Qg + (size_t)myq * rs + 64 * c + 32 * hi + 16);
        }
        lo ^= a.qsign;
        up ^= a.qsign;
        qf[c] = join(lo, up);
    }

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    // Swizzles: K rows (128 bytes) put chunk c of row r at c ^ ((r >> 1) & 7);
    // V^T rows (64 bytes) at c ^ ((r >> 2) & 3).
    auto swk = [](int row) { return (row >> 1) & 7; };
    auto swv = [](int row) { return (row >> 2) & 3; };
    auto kbuf = [&](int i) { return smem + i * TILE; };
    auto vbuf = [&](int i) { return smem + (2 + i) * TILE; };

    // Direct loads: wave load `inst` fills LDS bytes inst*1024 .. +1023; lane i
    // fetches the global chunk that the swizzle places in slot i. K runs one
    // tile ahead of V (tile t's scores are computed during step t - 1).
    auto dma_k = [&](int t, unsigned char* kd) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int inst = wave + NW * j;
            const int row = inst * (1024 / KRB) + lane / KCH;           // key row within the tile
            const int c = (lane % KCH) ^ swk(row);
            const int key = min(t * BN + row, N - 1);                   // past N: clamped, masked later
            __builtin_amdgcn_global_load_lds(Kg + (size_t)key * rs + 16 * c, (lds8_void_t*)(kd + inst * 1024), 16,
                                             0, 0);
        }
    };
    auto dma_v = [&](int t, unsigned char* vd) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int inst = wave + NW * j;
            const int row = inst * (1024 / VRB) + lane / 4;             // d row of V^T
            const int c = (lane % 4) ^ swv(row);
            __builtin_amdgcn_global_load_lds(Vg + (size_t)row * a.ldv + t * BN + 16 * c,
                                             (lds8_void_t*)(vd + inst * 1024), 16, 0, 0);
        }
    };
    auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // Per-lane LDS offsets of the operand reads (bytes within a tile).
    auto koff = [&](int kb, int c, int s) {      // K row 32 kb + l32, logical chunk 4 c + 2 hi + s
        const int row = kb * 32 + l32;
        return row * KRB + (((4 * c + 2 * hi + s) ^ swk(row)) << 4);
    };
    auto voff = [&](int db, int s) {             // V^T row 32 db + l32, logical chunk 2 hi + s
        const int row = db * 32 + l32;
        return row * VRB + (((2 * hi + s) ^ swv(row)) << 4);
    };
    auto kread = [&](const unsigned char* Ks, int kb, int c) {
        return join(*reinterpret_cast<const u32x4*>(Ks + koff(kb, c, 0)),
                    *reinterpret_cast<const u32x4*>(Ks + koff(kb, c, 1)));
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m = -INFINITY;   // running max of S * c2 for query myq (base-2 units)
    float l = 0.f;         // running sum over this lane's keys (other half added at the end)
    const float c2 = a.c2;

    // Score MFMA i of a tile: block i % 2, d chunk i / 2 (two chains).
    constexpr int NS = 2 * DC;
    auto scores = [&](f32x16 (&s)[2], const unsigned char* Ks) {
        i32x8 ka[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) ka[i] = kread(Ks, i % 2, i / 2);
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int i = 0; i < NS; ++i) s[i % 2] = mfma_fp8(ka[i], qf[i / 2], s[i % 2]);
    };

    // Step t: the score MFMAs of tile t + 1 run interleaved with the softmax
    // of tile t (mask, exact running max, rescale, then the exponentials,
    // row sums and E4M3 packing in NS parts, one after each MFMA), then the
    // PV MFMAs of tile t. Loads of K_{t+2} and V_{t+1} are in flight meanwhile.
    auto step = [&](int t, f32x16 (&scur)[2], f32x16 (&snext)[2], auto masked_c) {
        if (t + 2 < ntiles) dma_k(t + 2, kbuf(t & 1));
        if (t + 1 < ntiles) dma_v(t + 1, vbuf((t + 1) & 1));
        const unsigned char* Ks = kbuf((t + 1) & 1);   // K_{t+1} (stale past the last tile; unused)
        i32x8 ka[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) ka[i] = kread(Ks, i % 2, i / 2);
        fence();
        if constexpr (decltype(masked_c)::value) {
            // Key of element u of block kb is t*BN + kb*32 + 8*(u/4) + 4*hi + u%4.
            const int lim = CAUSAL ? min(N - 1, myq) : N - 1;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int thr = lim - (t * BN + kb * 32 + 4 * hi);
#pragma unroll
                for (int u = 0; u < 16; ++u) scur[kb][u] = (8 * (u >> 2) + (u & 3) > thr) ? -INFINITY : scur[kb][u];
            }
        }
        float mc[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 16; u += 2)
                mc[(u / 2) % 2] = __builtin_fmaxf(__builtin_fmaxf(mc[(u / 2) % 2], scur[kb][u]), scur[kb][u + 1]);
        const float mx = max_halves(__builtin_fmaxf(mc[0], mc[1])) * c2;
        // Exact running max: P <= 1 for the E4M3 rounding.
        const float mn = __builtin_fmaxf(m, mx);
        if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {
            const float alpha = exp2_fast(m - mn);   // m = -inf: 0 (nothing accumulated yet)
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m = mn;
        }
        const float mu = (m == -INFINITY) ? 0.f : m;
        fence();
        uint32_t pw[2][4];
        float ls[2] = {0.f, 0.f};
        // Part g (0 .. 7) of the softmax: elements 4 (g % 4) .. +3 of block g / 4.
        auto part = [&](int g) {
            const int kb = g / 4, gg = g % 4;
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_fast(__builtin_fmaf(scur[kb][4 * gg + e], c2, -mu));
                ls[g % 2] += p[e];
            }
            pw[kb][gg] = pack_e4m3x4(p[0], p[1], p[2], p[3]);
        };
        snext[0] = f32x16{};
        snext[1] = f32x16{};
        constexpr int PPM = 8 / NS;                    // softmax parts per score MFMA
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            snext[i % 2] = mfma_fp8(ka[i], qf[i / 2], snext[i % 2]);
            fence();
#pragma unroll
            for (int g = i * PPM; g < (i + 1) * PPM; ++g) part(g);
            fence();
        }
        l += ls[0] + ls[1];
        // Lane half 0 keeps block 0 and takes the other half's block-0 keys;
        // lane half 1 the same for block 1. Key 32*hi + j is then byte j.
        i32x8 pb;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const auto sw = __builtin_amdgcn_permlane32_swap(pw[0][g], pw[1][g], false, false);
            pb[2 * g] = (int)sw[0];
            pb[2 * g + 1] = (int)sw[1];
        }
        const unsigned char* Vs = vbuf(t & 1);
        i32x8 va[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
            va[db] = join(*reinterpret_cast<const u32x4*>(Vs + voff(db, 0)),
                          *reinterpret_cast<const u32x4*>(Vs + voff(db, 1)));
        if constexpr (decltype(masked_c)::value) {
            // Ragged last tile: byte j of this lane's 32 V^T bytes is key t*BN + 32*hi + j; bytes of keys
            // at or past N are the caller's padding. Their P is 0, but 0 times a NaN code is NaN, so they
            // are cleared in registers and the result does not depend on what the padding holds.
            const int valid = N - (t * BN + 32 * hi);
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int nb = valid - 4 * w;   // real bytes in dword w
                const uint32_t keep = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - nb))));
#pragma unroll
                for (int db = 0; db < DB; ++db) va[db][w] = (int)((uint32_t)va[db][w] & keep);
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma_fp8(va[db], pb, oacc[db]);
        fence();
        wait_dma();
        __syncthreads();
    };

    // Prologue: K_0, V_0 and K_1 into LDS, then the scores of tile 0.
    dma_k(0, kbuf(0));
    dma_v(0, vbuf(0));
    if (ntiles > 1) dma_k(1, kbuf(1));
    wait_dma();
    __syncthreads();
    f32x16 sa[2], sb[2];
    scores(sa, kbuf(0));
    __syncthreads();   // kbuf(0) receives K_2 in step 0

    // Tiles before t_split need no mask for any wave; the rest run the masked
    // variant. Under the causal mask a wave stops computing at the first tile
    // whose keys all follow its last query, but keeps issuing its share of
    // the loads and passing the barriers until the workgroup is done.
    const int t_split = min(CAUSAL ? q0 / BN : ntiles, (N % BN) ? ntiles - 1 : ntiles);
    auto idle = [&](int tt) { return CAUSAL && tt * BN > qw + 31; };
    int t = 0;
    for (; t + 1 < t_split; t += 2) {
        step(t, sa, sb, std::false_type{});
        step(t + 1, sb, sa, std::false_type{});
    }
    if (t < t_split) {
        step(t, sa, sb, std::false_type{});
        ++t;
        sa[0] = sb[0];
        sa[1] = sb[1];
    }
    for (; t < ntiles; t += 2) {
        if (idle(t)) break;
        step(t, sa, sb, std::true_type{});
        if (t + 1 < ntiles) {
            if (idle(t + 1)) {
                ++t;
                break;
            }
            step(t + 1, sb, sa, std::true_type{});
        }
    }
    for (; t < ntiles; ++t) {
        if (t + 2 < ntiles) dma_k(t + 2, kbuf(t & 1));
        if (t + 1 < ntiles) dma_v(t + 1, vbuf((t + 1) & 1));
        wait_dma();
        __syncthreads();
    }

    const float lt = sum_halves(l);
    const float inv = a.dv / lt;
    if (myq < N) {
        __bf16* orow = Og + (size_t)myq * rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hi;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                st8(orow + d0, w);
            }
        if (hi == 0) a.lse[(size_t)bh * N + myq] = (m + __builtin_log2f(lt)) * kLn2;
    }
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream) {
    if (d != 128) return hipErrorInvalidValue;
    // Four waves, two workgroups per CU (eight waves with one workgroup per CU
    // measured no faster without the mask and 5% slower with it).
    constexpr int NW = 4;
    const long long grid = (long long)((a.N + 32 * NW - 1) / (32 * NW)) * a.B * a.H;
    if (causal)
        hipLaunchKernelGGL((fwd_fp8_kernel<128, true, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_fp8_kernel<128, false, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fa
