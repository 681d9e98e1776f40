// micro.hip -- microbenchmarks of the gfx950 units the attention kernels
// depend on (C ABI in include/fa_micro.h). Each kernel keeps its results
// live through a vector store, so the compiler cannot drop the measured work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_micro.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kOk = 0, kInvalid = 1, kHip = 4;

__device__ __forceinline__ void stamp_begin(unsigned long long& t, unsigned long long& r) {
    t = __builtin_amdgcn_s_memtime();
    r = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void stamp_end(unsigned long long* clk, unsigned long long t0, unsigned long long r0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        unsigned long long* c = clk + 4 * (size_t)blockIdx.x;
        c[0] = t0;
        c[1] = t1;
        c[2] = r0;
        c[3] = r1;
    }
}

// Pseudo-random bf16 in [-2, 2) from an integer (a multiplicative hash).
__device__ __forceinline__ __bf16 rnd_bf16(uint32_t x) {
    x *= 0x9E3779B1u;
    x ^= x >> 15;
    x *= 0x85EBCA77u;
    x ^= x >> 13;
    return (__bf16)((float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f);
}

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

// Operand sources: MODE 0 -- one constant register pair (operand bits never
// change); MODE 1 -- eight register pairs of pseudo-random values used in
// turn (the multiplier inputs change every product, as with real data);
// MODE 2 -- the A operand of every product read from LDS (ds_read_b128,
// pseudo-random contents, conflict-free), B from registers as in MODE 1;
// MODE 3 -- both operands read from LDS (2 KB per product); MODE 4 / 5 -- as
// MODE 1, but with one / two accumulator chains instead of four (every
// product depends on the one issued one / two products earlier).
template <int MODE>
__global__ __launch_bounds__(256) void micro_mfma_bf16_kernel(float* out, unsigned long long* clk, int iters) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[64 * 1024 / 2];
    const int lane = threadIdx.x & 63;
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[r][i] = MODE == 0 ? (__bf16)((float)((lane + i) & 7) * 0.125f) : rnd_bf16(seed + 16 * r + i);
            b[r][i] = MODE == 0 ? (__bf16)((float)((lane * 3 + i) & 7) * 0.0625f) : rnd_bf16(seed + 16 * r + 8 + i);
        }
    if constexpr (MODE >= 2) {
        for (int i = threadIdx.x; i < 64 * 1024 / 2; i += 256) lds[i] = rnd_bf16(blockIdx.x * 65536u + i);
        __syncthreads();
    }
    // Wave w reads its own 16 KB quarter of the LDS, 1 KB per product.
    const int lbase = (threadIdx.x >> 6) * 8192 + lane * 8;
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    unsigned long long t0, r0;
    stamp_begin(t0, r0);
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            bf16x8 x = a[r];
            if constexpr (MODE >= 2) x = *(const lds_bf16x8_t*)(lds + lbase + ((it + r) & 15) * 512);
            bf16x8 y = MODE == 0 ? b[0] : b[r];
            if constexpr (MODE == 3) y = *(const lds_bf16x8_t*)(lds + lbase + ((it + r + 8) & 15) * 512);
            const bf16x8 xa = MODE == 0 ? a[0] : x;
            constexpr int NC = MODE == 4 ? 1 : MODE == 5 ? 2 : 4;   // accumulator chains
            if (r % NC == 0) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, y, c0, 0, 0, 0);
            if (r % NC == 1) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, y, c1, 0, 0, 0);
            if (r % NC == 2) c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, y, c2, 0, 0, 0);
            if (r % NC == 3) c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, y, c3, 0, 0, 0);
        }
    }
    stamp_end(clk, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// MFMAs interleaved with a wave's own VALU work: each MFMA (four chains, random
// register operands as in mode 1) is followed by NF independent v_fma_f32 and
// NE v_exp_f32 on eight other registers, fenced so the compiler keeps the
// order. Run with two workgroups of four waves per CU (two waves per SIMD),
// the attention kernels' occupancy; compare with the plain MFMA stream.
template <int NF, int NE>
__global__ __launch_bounds__(256, 2) void micro_mfma_valu_kernel(float* out, unsigned long long* clk, int iters) {
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[r][i] = rnd_bf16(seed + 16 * r + i);
            b[r][i] = rnd_bf16(seed + 16 * r + 8 + i);
        }
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.001f * (float)(threadIdx.x + j);
    const float cf = 0.999f, cb = 0.0001f;
    f32x16 c[4] = {};
    unsigned long long t0, r0;
    stamp_begin(t0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            c[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[r], c[r], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NF; ++k) v[k % 8] = __builtin_fmaf(v[k % 8], cf, cb);
#pragma unroll
            for (int k = 0; k < NE; ++k) v[(k + 4) % 8] = __builtin_amdgcn_exp2f(-v[(k + 4) % 8]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    stamp_end(clk, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += c[r][i];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void micro_exp2_kernel(float* out, unsigned long long* clk, int iters) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)(threadIdx.x & 63) + 0.1f * (float)j;
    unsigned long long t0, r0;
    stamp_begin(t0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    stamp_end(clk, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// One problem per 64-lane workgroup. Lane (r, h) = (lane % 32, lane / 32)
// supplies bytes 32h .. 32h+31 of row r of A_s and of column r of B_s; the
// accumulator element u of that lane is C[8 (u / 4) + 4 h + u % 4][r].
__global__ __launch_bounds__(64) void micro_fp8_dot_kernel(const unsigned char* a, const unsigned char* b, float* c,
                                                           int chain) {
    const int lane = threadIdx.x;
    const int r = lane & 31, h = lane >> 5;
    const size_t p = blockIdx.x;
    f32x16 acc = {};
    for (int s = 0; s < chain; ++s) {
        const size_t off = ((p * chain + s) * 32 + r) * 64 + 32 * h;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(a + off);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(a + off + 16);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(b + off);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(b + off + 16);
        const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
    }
    float* cp = c + p * 32 * 32;
#pragma unroll
    for (int u = 0; u < 16; ++u) cp[(8 * (u >> 2) + 4 * h + (u & 3)) * 32 + r] = acc[u];
}

__global__ __launch_bounds__(256) void micro_atomic_add_kernel(float* buf, int reps) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (int k = 0; k < reps; ++k) unsafeAtomicAdd(buf + i, 1.0f);
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int fa_micro_mfma_bf16(float* out, unsigned long long* clk, int blocks, int iters, int mode, hipStream_t stream) {
    if (!aligned16(out) || !aligned16(clk) || blocks < 1 || iters < 2 || iters > (1 << 24) || iters % 2 != 0)
        return kInvalid;
    if (mode == 0)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else if (mode == 1)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else if (mode == 2)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else if (mode == 3)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else if (mode == 4)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else if (mode == 5)
        hipLaunchKernelGGL(micro_mfma_bf16_kernel<5>, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    else
        return kInvalid;
    return hipGetLastError() == hipSuccess ? kOk : kHip;
}

int fa_micro_mfma_valu(float* out, unsigned long long* clk, int blocks, int iters, int nfma, int nexp,
                       hipStream_t stream) {
    if (!aligned16(out) || !aligned16(clk) || blocks < 1 || iters < 1 || iters > (1 << 24)) return kInvalid;
#define FA_MV(F, E)                                                                                          \
    if (nfma == F && nexp == E) {                                                                           \
        hipLaunchKernelGGL((micro_mfma_valu_kernel<F, E>), dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, \
                           iters);                                                                          \
        return hipGetLastError() == hipSuccess ? kOk : kHip;                                               \
    }
    FA_MV(0, 0) FA_MV(2, 0) FA_MV(4, 0) FA_MV(8, 0) FA_MV(0, 1) FA_MV(0, 2) FA_MV(0, 4) FA_MV(4, 2) FA_MV(6, 2)
#undef FA_MV
    return kInvalid;
}

int fa_micro_exp2(float* out, unsigned long long* clk, int blocks, int iters, hipStream_t stream) {
    if (!aligned16(out) || !aligned16(clk) || blocks < 1 || iters < 1 || iters > (1 << 24)) return kInvalid;
    hipLaunchKernelGGL(micro_exp2_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, clk, iters);
    return hipGetLastError() == hipSuccess ? kOk : kHip;
}

int fa_micro_fp8_dot(const void* a, const void* b, float* c, int problems, int chain, hipStream_t stream) {
    if (!aligned16(a) || !aligned16(b) || !aligned16(c) || problems < 1 || chain < 1 || chain > 64) return kInvalid;
    hipLaunchKernelGGL(micro_fp8_dot_kernel, dim3((unsigned)problems), dim3(64), 0, stream,
                       static_cast<const unsigned char*>(a), static_cast<const unsigned char*>(b), c, chain);
    return hipGetLastError() == hipSuccess ? kOk : kHip;
}

int fa_micro_atomic_add(float* buf, long long n, int reps, hipStream_t stream) {
    if (!aligned16(buf) || n < 256 || n % 256 != 0 || n / 256 >= (1LL << 31) || reps < 1) return kInvalid;
    hipLaunchKernelGGL(micro_atomic_add_kernel, dim3((unsigned)(n / 256)), dim3(256), 0, stream, buf, reps);
    return hipGetLastError() == hipSuccess ? kOk : kHip;
}

}  // extern "C"
