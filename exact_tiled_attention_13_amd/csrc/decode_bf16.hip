// decode_bf16.hip -- bf16 decoding against a key/value cache for gfx950.
//
// The pages separate the first pass over a context (prefill) from token-by-
// token generation (decoding), whose bottleneck differs (page "FlashAttention-2:
// atención eficiente en GPU para contextos largos", section "Cómo documentar
// una diferencia técnica"). Decoding computes the same exact attention for a
// few new query rows: query i is the token at position Nk - Nq + i, so under
// the causal mask it sees keys j <= Nk - Nq + i. With few query rows there is
// little arithmetic per cache byte, so the call is bound by streaming K and V
// from HBM, and the work is split over the key range (split-KV) to occupy the
// whole chip even at batch 1:
//
//   decode_split_kernel: one wave per (key chunk, K/V head, batch). The G * Nq
//     query rows that read this K/V head (at most 32) are the columns of one
//     32x32 MFMA block; the chunk's keys stream through LDS in tiles of 32
//     (direct-to-LDS loads, three stages, two tiles in flight) with the same
//     online softmax as the forward pass. It writes the chunk's O (normalised
//     within the chunk) and LSE, fp32, to the workspace; a row that sees no
//     key in the chunk gets O = 0 and LSE = -inf.
//   decode_merge_kernel: one workgroup per query row, LSE = ln sum_s exp(LSE_s) and
//     O = sum_s exp(LSE_s - LSE) O_s, the exact combination of the chunks
//     (the global normaliser built from per-block statistics, page section
//     "Bloques pequeños, normalización global").
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace fa {

// s_waitcnt operand that waits until at most n vector-memory operations are
// outstanding and leaves the export and LDS counters alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(vmcnt_only(0) == 0x0F70, "vmcnt(0) encoding");

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
    using T = LdsTile<D, 32>;
    constexpr int BN = T::ROWS;          // keys per tile
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    constexpr int RB = T::RB;
    constexpr int NST = 3;               // LDS stages (K and V each)
    constexpr int NL = 2 * T::NINST;     // direct loads per tile (K and V)
    static_assert(2 * NL <= 63, "two tiles in flight must fit the vmcnt counter");
    constexpr int kVmcntNL = vmcnt_only(NL);
    constexpr int kVmcnt2NL = vmcnt_only(2 * NL);
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * 2 * T::BYTES];
    lds_poison(smem, sizeof(smem));

    const int S = a.S, H = a.H, Hkv = a.Hkv, Nq = a.Nq, Nk = a.Nk, R = a.R;
    const int bh = blockIdx.x / S;
    const int s = blockIdx.x - bh * S;
    const int b = bh / Hkv, hk = bh - b * Hkv;
    const int G = H / Hkv;

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // This lane's query row (column of the score block) and its position.
    const int r = l32;
    const bool live = r < R;
    const int qi = live ? r / G : 0;
    const int qh = hk * G + (live ? r - (r / G) * G : 0);
    const int pos = Nk - Nq + qi;

    // Q row as the B operand of S^T = K Q^T (lane holds row r, d chunk
    // c*16 + hi*8 .. +8); padding rows are zero. The sign of a negative
    // scale is folded into Q, exponents use c2 = |scale| * log2(e).
    bf16x8 qf[DC];
    {
        const __bf16* qrow = static_cast<const __bf16*>(a.q) + (((size_t)b * Nq + qi) * H + qh) * D;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (live) x = ld16(qrow + c * 16 + hi * 8) ^ a.qsign;
            qf[c] = as_bf16x8(x);
        }
    }

    const size_t rskv = (size_t)Hkv * D;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + ((size_t)b * Nk * Hkv + hk) * D;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + ((size_t)b * Nk * Hkv + hk) * D;
    const int kbeg = s * a.L;
    const int kend = min(kbeg + a.L, Nk);
    const int ntiles = (kend - kbeg + BN - 1) / BN;
    const float c2 = a.c2;

    unsigned toff[T::NINST];
    T::template offsets<1>(toff, rskv, 0, lane);
    auto kst = [&](int i) { return smem + i * 2 * T::BYTES; };
    auto vst = [&](int i) { return smem + i * 2 * T::BYTES + T::BYTES; };
    // Rows past Nk are clamped to Nk - 1 by the loader and masked below.
    auto dma = [&](int t, unsigned char* __restrict__ kd, unsigned char* __restrict__ vd) {
        T::template load<1>(kd, Kg, rskv, kbeg + t * BN, Nk, 0, lane, toff);
        T::template load<1>(vd, Vg, rskv, kbeg + t * BN, Nk, 0, lane, toff);
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m = -INFINITY;                 // running max of this row, base-2 units
    float l = 0.f;                       // running sum over this lane's keys
    const int rowb = T::rowbase(lane);
    const int trb0 = T::trbase(lane, 0);
    const int trb1 = T::trbase(lane, 1);

    // One tile, with the current stage and the stage receiving tile t + 2 as
    // distinct restrict pointers: the LDS reads of tile t need not wait for
    // the loads in flight, which the explicit vmcnt wait below orders.
    auto step = [&](int t, const unsigned char* __restrict__ Ks, const unsigned char* __restrict__ Vs,
                    unsigned char* __restrict__ Kn, unsigned char* __restrict__ Vn, auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        // Wait for tile t's loads only: the NL loads of each later tile in
        // flight may stay outstanding.
        if (t + 2 < ntiles) {
            dma(t + 2, Kn, Vn);
            __builtin_amdgcn_s_waitcnt(kVmcnt2NL);
        } else if (t + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(kVmcntNL);
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        }
        __builtin_amdgcn_sched_barrier(0);
        // All operand reads of the tile are issued at once, K rows first: V's
        // transposing reads complete under the score MFMAs and the softmax.
        bf16x8 ka[DC], va[2][DB];
#pragma unroll
        for (int c = 0; c < DC; ++c) ka[c] = T::read_row(Ks, rowb ^ (c << 5));
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                va[kc][db] = T::read_tr(Vs, (trb0 ^ (db << 6)) + kc * 16 * RB, (trb1 ^ (db << 6)) + kc * 16 * RB);
        __builtin_amdgcn_sched_barrier(0);
        // S^T = K Q^T: 32 keys x 32 query rows.
        f32x16 sc = f32x16{};
#pragma unroll
        for (int c = 0; c < DC; ++c) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], sc, 0, 0, 0);
        // Element u holds key k0 + 8*(u/4) + 4*hi + u%4 of this lane's row.
        const int k0 = kbeg + t * BN;
        if constexpr (MASKED) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int key = k0 + 8 * (u >> 2) + 4 * hi + (u & 3);
                const bool vis = key < Nk && (!CAUSAL || key <= pos);
                sc[u] = vis ? sc[u] : -INFINITY;
            }
        }
        float mt = sc[0];
#pragma unroll
        for (int u = 1; u < 16; ++u) mt = __builtin_fmaxf(mt, sc[u]);
        mt = max_halves(mt) * c2;
        const float mn = __builtin_fmaxf(m, mt);
        const float mu = (mn == -INFINITY) ? 0.f : mn;   // no visible key yet: every p is 0
        const float alpha = exp2_fast(m - mu);
        m = mn;
        float p[16];
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            p[u] = exp2_fast(__builtin_fmaf(sc[u], c2, -mu));
            ls += p[u];
        }
        l = l * alpha + ls;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 16; ++u) oacc[db][u] *= alpha;
        // O^T += V^T P^T: the 8 keys of chunk kc this lane holds, in the order
        // of the transposing read's K index.
        bf16x8 pb[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * kc + 2 * e], p[8 * kc + 2 * e + 1]);
            pb[kc] = as_bf16x8(w);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kc][db], pb[kc], oacc[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    if (ntiles > 0) dma(0, kst(0), vst(0));
    if (ntiles > 1) dma(1, kst(1), vst(1));
    // Tiles that hold a key past Nk, or (causal) past the first query row's
    // position, take the masked path; every other tile is fully visible.
    const int first_masked = CAUSAL ? min(Nk, Nk - Nq + 1) : Nk;   // first key that some row cannot see
    int cs = 0;
    for (int t = 0; t < ntiles; ++t) {
        const int ns = cs == 0 ? 2 : cs - 1;                       // (t + 2) % 3
        if (kbeg + (t + 1) * BN <= first_masked)
            step(t, kst(cs), vst(cs), kst(ns), vst(ns), std::false_type{});
        else
            step(t, kst(cs), vst(cs), kst(ns), vst(ns), std::true_type{});
        cs = cs == 2 ? 0 : cs + 1;
    }

    const float lt = sum_halves(l);
    if (live) {
        const size_t row = ((size_t)bh * S + s) * R + r;
        float* orow = a.opart + row * D;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hi;
                const f32x4 w = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                                 oacc[db][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + d0) = w;
            }
        if (hi == 0) a.lpart[row] = lt > 0.f ? (m + __builtin_log2f(lt)) * kLn2 : -INFINITY;
    }
}

// One workgroup of 256 threads per query row: combine the row's S chunk
// results. The LSE reductions run over all threads (chunks s = t, t + 256,
// ...); for O, thread t takes 4 consecutive d (t % (D/4)) and the chunks
// s = t / (D/4) + k * (256 / (D/4)), and the partial sums meet in LDS.
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off);
        x = is_max ? __builtin_fmaxf(x, y) : x + y;
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();                     // red may still be read by the previous reduction
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    const float a = red[0], b = red[1], c = red[2], d = red[3];
    return is_max ? __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d)) : (a + b) + (c + d);
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int TPR = D / 4;           // threads per d range
    constexpr int SG = 256 / TPR;        // chunk groups
    __shared__ f32x4 part[SG][TPR];
    __shared__ float red[4];
    lds_poison(part, sizeof(part));
    lds_poison(red, sizeof(red));
    const int t = threadIdx.x;
    const long long row = blockIdx.x;    // (b, i, h)
    const int h = (int)(row % a.H);
    const int i = (int)((row / a.H) % a.Nq);
    const int b = (int)(row / ((long long)a.H * a.Nq));
    const int G = a.H / a.Hkv;
    const int hk = h / G;
    const int r = i * G + (h - hk * G);
    const int S = a.S;
    const size_t p0 = ((size_t)b * a.Hkv + hk) * S * a.R + r;         // chunk s at p0 + s * R
    float mx = -INFINITY;
    for (int s = t; s < S; s += 256) mx = __builtin_fmaxf(mx, a.lpart[p0 + (size_t)s * a.R]);
    mx = block_reduce(mx, true, red);
    float lse = -INFINITY;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    const int c = t % TPR, sg = t / TPR;
    if (mx != -INFINITY) {                // (uniform over the block)
        float sum = 0.f;
        for (int s = t; s < S; s += 256) sum += __expf(a.lpart[p0 + (size_t)s * a.R] - mx);
        sum = block_reduce(sum, false, red);
        lse = mx + __logf(sum);
        for (int s = sg; s < S; s += SG) {
            const size_t ps = p0 + (size_t)s * a.R;
            const float w = __expf(a.lpart[ps] - lse);
            const f32x4 x = *reinterpret_cast<const f32x4*>(a.opart + ps * D + 4 * c);
            o += w * x;
        }
    }
    part[sg][c] = o;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
        for (int k = 1; k < SG; ++k) o += part[k][c];
        u32x2 packed;
        packed[0] = pack_bf16x2(o[0], o[1]);
        packed[1] = pack_bf16x2(o[2], o[3]);
        st8(static_cast<__bf16*>(a.o) + (((size_t)b * a.Nq + i) * a.H + h) * D + 4 * c, packed);
        if (c == 0) a.lse[((size_t)b * a.H + h) * a.Nq + i] = lse;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
    const long long g = (long long)a.S * a.Hkv * a.B;
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL>), dim3((unsigned)g), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Nq * a.H;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)rows), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch_dec<128, true>(a, stream) : launch_dec<128, false>(a, stream);
    return causal ? launch_dec<64, true>(a, stream) : launch_dec<64, false>(a, stream);
}

}  // namespace fa
