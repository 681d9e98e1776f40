// common.hpp -- shared device helpers of libfa_mi355x (gfx950 only).
//
// Vector types for the CDNA4 matrix-core builtins, the launch-argument
// structs, the workgroup -> (tile, head, batch) map and small lane helpers.
// Every kernel in this library includes this header; nothing here is used by
// the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Launch arguments of the forward kernels. Tensors are [B, N, H, d] with d
// fastest; lse is [B, H, N].
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N;
    int Hkv;          // K/V heads (H is a multiple; query head h reads K/V head h / (H / Hkv))
    float c2;         // |scale| * log2(e): scores are exponentiated in base 2
    uint32_t qsign;   // 0x80008000 when scale < 0 (folded into Q's sign bits), else 0
    float qsign_f;    // -1.0f when scale < 0, else 1.0f (fp32 kernels)
};

// Launch arguments of the backward kernels.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* dd;        // workspace: -D_i = -dO_i . O_i, fp32 [B, H, Npad]
    float* lse2;      // workspace: LSE_i * log2(e), fp32 [B, H, Npad] (+inf on padded rows)
    float* part;      // workspace: fp32 partial dK (unscaled), dV [gsplit][2][B, N, Hkv, d], when gsplit > 1
    int gsplit;       // grouped-query dK/dV: query heads of a K/V head split over this many workgroups
    int B, H, N;
    int Hkv;          // K/V heads, as in FwdArgs (k, v, dk, dv are [B, N, Hkv, d])
    float scale;      // the caller's scale (multiplies dQ and dK)
    float c2;         // |scale| * log2(e)
    uint32_t qsign;   // as in FwdArgs
};

// Launch arguments of the FP8 forward. q, k are E4M3 bytes [B, N, H, d]; vt is
// V transposed per head, E4M3 bytes [B, H, d, ldv] (keys contiguous, keys N ..
// ldv-1 of each row finite padding); o bf16 [B, N, H, d]; lse [B, H, N].
struct Fp8Args {
    const void* q;
    const void* k;
    const void* vt;
    void* o;
    float* lse;
    int B, H, N;
    int ldv;          // bytes per V^T row, a multiple of 64 and at least N
    float c2;         // |scale * q_descale * k_descale| * log2(e)
    uint32_t qsign;   // 0x80808080 when that product is negative (folded into Q's sign bits), else 0
    float dv;         // V descale: O = (P V8) * dv / l
};

// Launch arguments of the decoding kernels. q, o are [B, Nq, H, d]; k, v the
// cache [B, Nk, Hkv, d]; lse [B, H, Nq]. Query row r (0 <= r < R) of K/V head
// hk is query i = r / G of head hk * G + r % G, G = H / Hkv.
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* opart;     // workspace: per-chunk outputs, fp32 [B, Hkv, S, R, d]
    float* lpart;     // workspace: per-chunk LSE (natural log), fp32 [B, Hkv, S, R]
    int B, H, Hkv, Nq, Nk;
    int R;            // query rows per K/V head, G * Nq (at most 32)
    int S;            // key chunks
    int L;            // keys per chunk (a multiple of 32); chunk s is keys s*L .. min((s+1)*L, Nk)-1
    float c2;         // as in FwdArgs
    uint32_t qsign;   // as in FwdArgs
};

// Race check. In the build with -DFA_LDS_POISON=1 every kernel calls this on
// each of its LDS arrays before anything else: the workgroup fills the array
// with 0xFF bytes (a NaN in fp32 and in bf16) and waits at a barrier, so a
// read of LDS that none of the kernel's loads or stores wrote carries NaN
// into the results (even a probability of zero times NaN is NaN). In the
// normal build it compiles to nothing. `bytes` is a multiple of 4 and `p` is
// 4-byte aligned.
__device__ __forceinline__ void lds_poison(void* p, int bytes) {
#if defined(FA_LDS_POISON) && FA_LDS_POISON
    uint32_t* w = static_cast<uint32_t*>(p);
    for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
    __syncthreads();
#else
    (void)p;
    (void)bytes;
#endif
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Remap the dispatch index so that XCD x receives a contiguous range of
// logical tile indices: the query blocks of one head then run on one XCD at
// the same time and share that head's K/V tiles in its L2. Bijective on
// [0, total).
__device__ __forceinline__ int xcd_remap(int id, int total) {
    constexpr int kXcd = 8;
    const int per = total / kXcd;
    const int rem = total % kXcd;
    const int x = id % kXcd;
    const int k = id / kXcd;
    return x * per + (x < rem ? x : rem) + k;
}

// Work item of workgroup `id` in a grid of `units` x `nb` items: a unit is a
// head (or a K/V head and part of its query-head group), and its nb blocks
// are its query or key blocks. XCD x gets a contiguous range of items
// (xcd_remap), so the units of that range run on one XCD and share its L2.
// blk is the block's rank in the order the XCD should start them. Without the
// causal mask every block costs the same and a unit's blocks run together
// (unit-major). Under the mask (ranked), rank 0 is the heaviest block; when
// the units split evenly over the 8 XCDs, each XCD starts its units'
// blocks rank-major -- the heaviest block of every unit first -- so that its
// CUs get the work longest-first. Unit by unit instead, with several units per
// XCD, the heavy blocks of an XCD's last unit start only after the light ones
// of the others and finish alone, leaving the other CUs idle.
__device__ __forceinline__ void work_item(int id, int nb, int units, bool ranked, int& unit, int& blk) {
    const int r = xcd_remap(id, nb * units);
    if (ranked && (units & 7) == 0) {
        const int ux = units >> 3;       // units per XCD
        const int per = ux * nb;
        const int x = r / per, j = r - x * per;
        blk = j / ux;
        unit = x * ux + (j - blk * ux);
    } else {
        unit = r / nb;
        blk = r - unit * nb;
    }
}

// Combine a per-lane value with the one held by lane (lane ^ 32): in the
// 32x32 accumulator layout the two halves of a wave64 hold the same column.
// v_permlane32_swap exchanges the upper 32 lanes of one operand with the
// lower 32 lanes of the other; with x in both, each lane ends up holding x of
// its own lane and of lane ^ 32, one in each result. It runs on the VALU (a
// shuffle through ds_bpermute would count as an LDS access and wait for any
// direct-to-LDS loads in flight). max and + are commutative, so both halves
// get bit-identical results.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3:
// 32-bit elements, no swizzle, no stride). Loads through it take a per-lane
// 32-bit offset and a uniform offset held in an SGPR, so a tile load whose
// per-lane offsets repeat from tile to tile needs no per-lane address
// arithmetic (a 64-bit address per lane costs a VALU add per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Materialises x in a VGPR at this point of the program: the computation of x
// can no longer be sunk past it (the value itself is unchanged). Used to keep
// running sums spread over a hand-scheduled loop instead of being gathered
// into one serial chain at their first use.
__device__ __forceinline__ void pin_vgpr(float& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}
__device__ __forceinline__ void pin_vgpr(int& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}
__device__ __forceinline__ void pin_vgpr(uint32_t& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}

// Round-to-nearest-even fp32 pair -> packed bf16 pair (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// 16-byte global load / store helpers on raw bf16 bits.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ void st16f(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Transpose four 8-element bf16 rows (keys r0..r3, 8 consecutive d each) into
// eight 4-element columns: out[c] holds (r0[c], r1[c], r2[c], r3[c]) as two
// dwords, for c = 0..7.
__device__ __forceinline__ void transpose_4x8(const u32x4 (&r)[4], u32x2 (&out)[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a = r[0][w], b = r[1][w], c = r[2][w], d = r[3][w];
        // even element (low halves), odd element (high halves)
        out[2 * w][0] = (a & 0xffffu) | (b << 16);
        out[2 * w][1] = (c & 0xffffu) | (d << 16);
        out[2 * w + 1][0] = (a >> 16) | (b & 0xffff0000u);
        out[2 * w + 1][1] = (c >> 16) | (d & 0xffff0000u);
    }
}

// Position of tile-local key k inside a V^T / K^T row. Within each 16-key
// chunk the keys are stored as [0-3, 8-11, 4-7, 12-15] so that the 8 keys
// one lane half contributes to a 32x32x16 MFMA (keys 4h..4h+3 and
// 8+4h..8+4h+3, the order a 32x32 accumulator holds them in) are one
// contiguous 16-byte read. k must be a multiple of 4; returns the position of
// the group k..k+3.
__device__ __forceinline__ int kperm4(int k) {
    const int g = (k >> 2) & 3;
    return (k & ~15) + ((g & 1) << 3) + ((g >> 1) << 2);
}

}  // namespace fa
