// fwd_fp32.hip -- fp32 forward of exact tiled attention for gfx950.
//
// Same method as the bf16 forward (online softmax over K/V tiles staged in
// LDS, one wavefront per 32 query rows, causal tiles above the diagonal
// skipped, masking only on diagonal and tail tiles; page "FlashAttention-2:
// atención eficiente en GPU para contextos largos", sections "Bloques
// pequeños, normalización global" and "Tres mejoras en la utilización de la
// GPU"), with every operand and product in fp32: v_mfma_f32_32x32x2_f32 for
// S^T = K Q^T and O^T += V^T P^T, and no rounding below fp32 anywhere. This
// variant exists for fp32 callers and for tight-tolerance checks; it is
// single-buffered and not tuned.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_fp32_kernel(FwdArgs a) {
    constexpr int BM = 128;
    constexpr int BN = 32;
    constexpr int KS = D + 1;   // odd stride: the 32 lanes reading one column hit 32 banks
    constexpr int VS = D + 8;   // rows 4 apart land in opposite bank halves
    constexpr int DB = D / 32;
    __shared__ float Ks[BN * KS];
    __shared__ __attribute__((aligned(16))) float Vs[BN * VS];
    lds_poison(Ks, sizeof(Ks));
    lds_poison(Vs, sizeof(Vs));

    const int B = a.B, H = a.H, N = a.N;
    const int nq = (N + BM - 1) / BM;
    int bh, qb;
    work_item(blockIdx.x, nq, B * H, CAUSAL, bh, qb);
    if (CAUSAL) qb = nq - 1 - qb;         // longest rows first
    const int b = bh / H, h = bh - b * H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const size_t rs = (size_t)H * D;
    const size_t base = ((size_t)b * N * H + h) * D;
    const float* Qg = static_cast<const float*>(a.q) + base;
    const float* Kg = static_cast<const float*>(a.k) + base;
    const float* Vg = static_cast<const float*>(a.v) + base;
    float* Og = static_cast<float*>(a.o) + base;

    const int q0 = qb * BM;
    const int qw = q0 + wave * 32;
    const int myq = qw + l32;

    // Q^T (B operand of the 32x32x2 product): step c covers d = 2c + hi.
    float qf[D / 2];
#pragma unroll
    for (int c = 0; c < D / 2; ++c) qf[c] = (myq < N) ? a.qsign_f * Qg[(size_t)myq * rs + 2 * c + hi] : 0.f;

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m = -INFINITY, l = 0.f;
    const float c2 = a.c2;

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * BN;
        for (int id = tid; id < BN * D / 4; id += 256) {
            const int row = id / (D / 4), col = (id % (D / 4)) * 4;
            const int key = j0 + row;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < N) {
                kv = *reinterpret_cast<const f32x4*>(Kg + (size_t)key * rs + col);
                vv = *reinterpret_cast<const f32x4*>(Vg + (size_t)key * rs + col);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ks[row * KS + col + e] = kv[e];
            *reinterpret_cast<f32x4*>(Vs + row * VS + col) = vv;
        }
        __syncthreads();

        const bool active = !CAUSAL || (j0 <= qw + 31);
        if (active) {
            f32x16 s = f32x16{};
#pragma unroll
            for (int c = 0; c < D / 2; ++c)
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * KS + 2 * c + hi], qf[c], s, 0, 0, 0);

            const bool masked = (CAUSAL && j0 + BN - 1 > qw) || (j0 + BN > N);
            uint32_t dead = 0u;
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int key = j0 + 8 * (u >> 2) + 4 * hi + (u & 3);
                const bool kill = masked && (key >= N || (CAUSAL && key > myq));
                dead |= (kill ? 1u : 0u) << u;
                if (!kill) mx = __builtin_fmaxf(mx, s[u]);
            }
            mx = max_halves(mx);
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
            const float mnew = __builtin_fmaxf(m, mt);
            const float alpha = exp2_fast(m - mnew);
            m = mnew;
            float p[16];
            float rowsum = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                p[u] = ((dead >> u) & 1u) ? 0.f : exp2_fast(__builtin_fmaf(s[u], c2, -mnew));
                rowsum += p[u];
            }
            l = l * alpha + rowsum;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                oacc[db] *= alpha;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int key = 8 * (u >> 2) + 4 * hi + (u & 3);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VS + db * 32 + l32], p[u], oacc[db], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    const float lt = sum_halves(l);
    const float inv = 1.0f / lt;
    if (myq < N) {
        float* orow = Og + (size_t)myq * rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                           oacc[db][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) a.lse[(size_t)bh * N + myq] = (m + __builtin_log2f(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int nq = (a.N + 127) / 128;
    const long long grid = (long long)nq * a.B * a.H;
    hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_fp32(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
