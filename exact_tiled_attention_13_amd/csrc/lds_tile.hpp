// lds_tile.hpp -- LDS staging of 64-row bf16 tiles for the backward kernels.
//
// A tile is ROWS (64 unless stated) rows of one head's [*, d] slice (row stride H*d elements in
// global memory), stored in LDS unpadded, RB = 2d bytes per row, with the
// 16-byte chunks of each row permuted by an XOR swizzle f(row). The swizzle is
// chosen so that both access patterns the MFMA operands need are free of LDS
// bank conflicts:
//   * row reads (ds_read_b128): 16 consecutive rows at one chunk column;
//   * transposing reads (ds_read_b64_tr_b16): 4 consecutive rows x 64 bytes.
// Tiles are filled with direct-to-LDS loads (global_load_lds_dwordx4): one
// wave instruction writes 1 KB of LDS, lane i its 16-byte slot i, so each lane
// fetches the global chunk that the swizzle places in its slot.
#pragma once

#include "common.hpp"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// One 16-byte-per-lane direct-to-LDS load through a buffer resource over
// `bytes` bytes at `base`: lane i's 16 bytes at byte offset voff + soff land
// in LDS slot i of the 1 KB at dst.
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t bytes, unsigned char* dst, uint32_t voff,
                                                  uint32_t soff) {
    const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(base, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}

template <int D, int ROWS_ = 64>
struct LdsTile {
    static_assert(ROWS_ % 16 == 0, "tiles are whole 16-row swizzle groups");
    static constexpr int ROWS = ROWS_;
    static constexpr int RB = D * 2;            // bytes per row
    static constexpr int BYTES = ROWS * RB;     // bytes per tile
    static constexpr int NINST = BYTES / 1024;  // direct-to-LDS wave loads per tile
    static constexpr int RPI = 1024 / RB;       // rows per such load
    static constexpr int CPR = RB / 16;         // 16-byte chunks per row

    // Chunk permutation of row r (4 bits for d = 128, 3 bits for d = 64).
    __device__ static __forceinline__ int swz(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }

    // Element offsets (tile row * rs + chunk) of the chunks that lane `lane`
    // of wave `w` (of NW) fetches; they are the same for every tile, so a
    // kernel computes them once.
    template <int NW>
    __device__ static __forceinline__ void offsets(unsigned (&off)[NINST / NW], size_t rs, int w, int lane) {
        static_assert(NINST % NW == 0, "tile loads must split evenly over the waves");
#pragma unroll
        for (int j = 0; j < NINST / NW; ++j) {
            const int row = (w + NW * j) * RPI + lane / CPR;
            const int c = (lane % CPR) ^ swz(row);
            off[j] = (unsigned)row * (unsigned)rs + 8u * (unsigned)c;
        }
    }

    // Wave `w` of NW loads its share of rows row0 .. row0+63 of g (row
    // stride rs elements) into the tile at `dst`; `off` comes from offsets().
    // Rows at or past n are clamped to n - 1: callers mask them. Full tiles
    // only add the uniform row0 * rs to the precomputed offsets.
    template <int NW>
    __device__ static __forceinline__ void load(unsigned char* dst, const __bf16* g, size_t rs, int row0, int n,
                                                int w, int lane, const unsigned (&off)[NINST / NW]) {
        if (row0 + ROWS <= n) {
            const __bf16* gt = g + (size_t)row0 * rs;
#pragma unroll
            for (int j = 0; j < NINST / NW; ++j)
                __builtin_amdgcn_global_load_lds(gt + (size_t)off[j], (lds_void_t*)(dst + (w + NW * j) * 1024), 16,
                                                 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < NINST / NW; ++j) {
                const int inst = w + NW * j;
                const int row = inst * RPI + lane / CPR;
                const int c = (lane % CPR) ^ swz(row);
                const int grow = min(row0 + row, n - 1);
                __builtin_amdgcn_global_load_lds(g + (size_t)grow * rs + c * 8, (lds_void_t*)(dst + inst * 1024),
                                                 16, 0, 0);
            }
        }
    }

    // The same through a buffer resource over `bytes` bytes of g's rows (row
    // stride rs): whole tiles add the uniform row0 * rs in an SGPR to each
    // lane's fixed offset, with no per-lane address arithmetic; the ragged
    // last tile takes load()'s clamped path. A head's rows span less than
    // 2^32 bytes, so the 32-bit offsets hold. (The resource is rebuilt from
    // uniform values at each call; the compiler keeps it in SGPRs.)
    template <int NW>
    __device__ static __forceinline__ void load_buf(unsigned char* dst, const __bf16* g, uint32_t bytes, size_t rs,
                                                    int row0, int n, int w, int lane,
                                                    const unsigned (&off)[NINST / NW]) {
        if (row0 + ROWS <= n) {
            const uint32_t so = (uint32_t)row0 * (uint32_t)rs * 2u;
#pragma unroll
            for (int j = 0; j < NINST / NW; ++j) buffer_load_lds16(g, bytes, dst + (w + NW * j) * 1024, off[j] * 2u, so);
        } else {
            load<NW>(dst, g, rs, row0, n, w, lane, off);
        }
    }

    // Bytes of a head's rows 0 .. n-1 (row stride rs elements) from its first element.
    __device__ static __forceinline__ uint32_t span(size_t rs, int n) {
        return (uint32_t)(((size_t)(n - 1) * rs + D) * 2);
    }

    // Row reads: A/B operand of a 32x32x16 MFMA whose 32 rows are tile rows
    // rb*32 + lane%32 and whose K step cc covers d = cc*16 + (lane/32)*8 .. +8.
    // Byte offset = rowbase(lane) ^ (cc << 5), plus rb*32*RB.
    __device__ static __forceinline__ int rowbase(int lane) {
        const int l32 = lane & 31, hi = lane >> 5;
        const int f = swz(l32);
        return l32 * RB + ((hi ^ (f & 1)) << 4) + ((f >> 1) << 5);
    }

    // Transposing reads: the 32x16 operand whose rows are d = db*32 + lane%32
    // and whose K index runs over tile rows kc*16 + {4h..4h+3, 8+4h..8+4h+3}
    // (h = lane/32), as two ds_read_b64_tr_b16 (half 0: first four rows,
    // half 1: rows +8). Byte offset = trbase(lane, half) ^ (db << 6), plus
    // kc*16*RB.
    __device__ static __forceinline__ int trbase(int lane, int half) {
        const int g = lane >> 4, i = lane & 15, hi = lane >> 5;
        const int row = 4 * hi + (i >> 2) + 8 * half;            // row within the 16-row chunk
        const int f = swz(row);
        const int x = 2 * (g & 1) + ((i & 3) >> 1);               // 16-byte chunk within the 64-byte run
        return row * RB + ((f >> 2) << 6) + ((x ^ (f & 3)) << 4) + ((i & 1) << 3);
    }

    __device__ static __forceinline__ bf16x8 read_row(const unsigned char* t, int off) {
        return *reinterpret_cast<const bf16x8*>(t + off);
    }

    __device__ static __forceinline__ bf16x8 read_tr(const unsigned char* t, int off0, int off1) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(t + off0));
        const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(t + off1));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// ---------------------------------------------------------------------------
// Output rows through LDS. In a 32x32 accumulator whose columns are 32 rows
// of an output (lane % 32) and whose rows are d (block db), lane (l32, hi)
// holds elements db*32 + 8g + 4hi .. +3 of row l32 for g = 0..3.
// stage_rows packs them (times sc) to bf16 and writes them to a 32-row LDS
// region, 16-byte chunks of a row XOR-swizzled by the row; store_rows reads
// back whole 16-byte chunks and writes rows r0 .. r0+31 (those below n) of
// g (row stride rs elements), so that each store instruction covers
// contiguous rows instead of 8 bytes of 32 rows. The region belongs to one
// wave; LDS operations of a wave run in order, so no barrier is needed
// between the two.
template <int D>
__device__ __forceinline__ void stage_rows(unsigned char* sw, const f32x16 (&acc)[D / 32], float sc, int l32,
                                           int hi) {
    constexpr int RB = D * 2, CPR = RB / 16;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc);
            w[1] = pack_bf16x2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
            *reinterpret_cast<u32x2*>(sw + l32 * RB + (((db * 4 + g) ^ (l32 & (CPR - 1))) << 4) + 8 * hi) = w;
        }
}

template <int D>
__device__ __forceinline__ void store_rows(__bf16* g, size_t rs, const unsigned char* sw, int r0, int n,
                                           int lane) {
    constexpr int RB = D * 2, CPR = RB / 16;
#pragma unroll
    for (int j = 0; j < 32 * CPR / 64; ++j) {
        const int i = j * 64 + lane;
        const int row = i / CPR, ch = i % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sw + row * RB + ((ch ^ (row & (CPR - 1))) << 4));
        if (r0 + row < n) st16(g + (size_t)(r0 + row) * rs + ch * 8, v);
    }
}

}  // namespace fa
