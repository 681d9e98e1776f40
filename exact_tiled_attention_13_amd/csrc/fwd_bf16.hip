// fwd_bf16.hip -- bf16 forward of exact tiled attention for gfx950.
//
// Method (page "FlashAttention-2: atención eficiente en GPU para contextos
// largos"):
//   * section "Bloques pequeños, normalización global": K/V are streamed in
//     tiles through on-chip memory (LDS) and an online softmax keeps a running
//     row maximum m and row sum l, rescaling the partial output, so the N x N
//     score and probability matrices never reach HBM;
//   * section "Tres mejoras en la utilización de la GPU": the grid covers
//     (query block, head, batch), so a single long sequence still fills the
//     chip; each wavefront owns its own 32 query rows and all eight wavefronts
//     of a workgroup share the K/V tiles in LDS, so no partial output is ever
//     exchanged between wavefronts; tiles entirely above the causal diagonal
//     are never loaded, masking runs only on diagonal and ragged-tail tiles,
//     and the division by the row sum happens once, at the end.
//
// CDNA4 mapping (one wavefront = 64 lanes, 32 query rows):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K tile rows from LDS,
//                 B = Q^T held in VGPRs for the whole kernel. In the 32x32
//                 accumulator each lane holds one query column (lane % 32) and
//                 16 keys, so the row max / row sum are in-lane plus one
//                 exchange with lane ^ 32.
//   In the 8-wave form (long sequences, see kFwdShortN) waves 4-7 run half
//   a step behind waves 0-3 (ping-pong), and a tile's row maximum is only
//   taken when its probabilities outgrow the running one (kSumLimit below).
//   O^T += V^T P^T  A = V^T tile from LDS (stored transposed, keys permuted
//                 within 16-key chunks to the order the accumulator holds
//                 them in), B = P^T converted in registers from the S^T
//                 accumulator. The O^T accumulator again has one query per
//                 lane, so the online-softmax rescale is a per-lane scalar.
//   Softmax in base 2: p = exp2(S * c2 - m) with c2 = |scale| * log2(e); a
//   negative scale is folded into the sign bits of Q.
//   K/V tiles are fetched into LDS by direct-to-LDS loads (16 bytes per
//   lane) one step ahead of their use, double-buffered (V in four buffers in
//   the 8-wave ping-pong form); one barrier per tile.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {

// Online-softmax bookkeeping: the running maximum m is only moved when a
// tile's maximum exceeds it by more than kTau (base-2 units). Between moves the
// exponentials are taken against the stale m, so they stay below 2^kTau, and
// the final O / l and LSE = m + log2(l) are unchanged: the result is the same
// exact softmax, with the rescale of l and O skipped for most tiles.
constexpr float kTau = 8.0f;

// In the 8-wave form a tile's exponentials are taken against the running
// maximum m before the tile's own maximum is known. While every partial row
// sum of a tile (one lane's 32 keys) stays at or below kSumLimit, every
// probability is at most kSumLimit, far inside fp32 and bf16 range, and m
// stays. A partial sum
// above the limit (or not finite) sends the wave through the rescale path:
// the tile's scores are formed again (from K in global memory; the tile's
// LDS buffer is already being refilled), m moves to their maximum, l and O
// are rescaled, and the tile's probabilities are taken again. Which m is
// used changes no result but rounding: O / l and LSE = m + log2(l) are the
// same exact softmax. The first tile's maximum is taken before the loop.
constexpr float kSumLimit = 65536.0f;

// d = 128 sequences up to this length use 4-wave workgroups (see
// fwd_bf16_kernel), longer ones the 8-wave ping-pong form, which wins
// beyond 1024 tokens (measured on MI355X: 4-7% at 1500-2048 tokens without
// the mask, 7% at 1536 with it, 4-8% at 2730-4096; at 512-1024 tokens the
// two are level within 2%).
constexpr int kFwdShortN = 1024;
// d = 64 uses the 8-wave form from this length on, when its grid gives every
// CU at least two workgroups (kFwdMinWgs8): 5-6% faster without the mask and
// 2-10% with it at 4096-16384 tokens. Below, or on smaller grids, the 4-wave
// form with three workgroups per CU is faster (13% at 3000 tokens on 384
// 8-wave workgroups; level at 2048).
constexpr int kFwdShortN64 = 4096;
constexpr long long kFwdMinWgs8 = 512;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 1 : (D == 64 ? 3 : 2)) void fwd_bf16_kernel(FwdArgs a) {
    // NW waves per workgroup: 8 (two per SIMD, one workgroup per CU), or 4
    // with two workgroups sharing a CU (three at d = 64, within 168 VGPRs
    // and 48 KB of LDS each), so that one's start-up and tail overlap the
    // others' main loops and causal query blocks are shorter. (Three d = 64
    // workgroups per CU: 8-10% faster causal at 512-1024 tokens, 2-3%
    // without the mask, level at 16k tokens.)
    constexpr int BM = NW * 32;           // query rows per workgroup
    constexpr int BN = 64;                // keys per tile
    constexpr int RB = D * 2;             // bytes per K/V row
    constexpr int TILE = BN * RB;         // bytes per K or V tile
    constexpr int NINST = TILE / 1024;    // 1 KB direct-to-LDS wave loads per tile
    // Ping-pong (8 waves, the workgroup alone on its CU): waves
    // 4-7 run half a step behind waves 0-3 (see the main loop), so that on
    // each SIMD, which holds one wave of each half, one wave's exponentials
    // overlap the other's P V products instead of both waves reaching the
    // same phase together after every barrier. Waves 0-3 issue all the tile
    // loads.
    constexpr bool PP = NW == 8;
    constexpr int NL = PP ? NW / 2 : NW;  // waves that issue the tile loads
    constexpr int IPW = NINST / NL;       // ... per loading wave
    constexpr int RPI = 1024 / RB;        // rows covered by one such load
    constexpr int CPR = RB / 16;          // 16-byte chunks per row
    constexpr int DC = D / 16;            // 16-wide d chunks (MFMA K steps of S)
    constexpr int KB = BN / 32;           // 32-key blocks per tile
    constexpr int DB = D / 32;            // 32-wide d blocks of O^T
    static_assert(IPW * NL == NINST && IPW >= 1, "tile must split evenly over the waves");
    // V buffers: tile j in slot j % NVB. The ping-pong form needs three at a
    // time (V_{t-1}, V_t read while V_{t+1} arrives); four keep the slot a
    // compile-time constant in a loop body unrolled over U = 4 steps.
    constexpr int NVB = PP ? 4 : 2;
    constexpr int U = PP ? 4 : 2;

    // LDS: Kbuf[0], Kbuf[1], Vbuf[0 .. NVB-1]; rows unpadded, 16-byte chunks
    // XOR-swizzled per row (see swk / swv) so that the MFMA operand reads are
    // free of bank conflicts.
    // Q enters through LDS as well (see below) where the extra LDS still
    // leaves the workgroup's occupancy unchanged: at d = 64 (80 KB for the
    // 8-wave form, alone on its CU), not at d = 128, whose four-wave
    // workgroups already take 128 KB per CU and eight-wave ones 96 KB.
    constexpr bool QLDS = D == 64;
    constexpr int QST = QLDS ? NW * 32 * RB : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[(2 + NVB) * TILE + QST];
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

    const size_t rs = (size_t)H * D;                       // Q / O row stride (elements)
    const size_t base = ((size_t)b * N * H + h) * D;       // (b, 0, h, 0)
    // K / V head of this query head (grouped-query attention when Hkv < H).
    const int hk = h / (H / a.Hkv);
    const size_t rskv = (size_t)a.Hkv * D;                 // K / V row stride
    const size_t kvbase = ((size_t)b * N * a.Hkv + hk) * D;
    const __bf16* Qg = static_cast<const __bf16*>(a.q) + base;
    const __bf16* Kg = static_cast<const __bf16*>(a.k) + kvbase;
    const __bf16* Vg = static_cast<const __bf16*>(a.v) + kvbase;
    __bf16* Og = static_cast<__bf16*>(a.o) + base;

    const int q0 = qb * BM;
    const int qw = q0 + wave * 32;        // first query row of this wave
    const int myq = qw + l32;             // query row owned by this lane

    // Q^T fragments (B operand): lane holds Q[myq][c*16 + hi*8 .. +8].
    // With QLDS each wave first copies its 32 rows into its own LDS region
    // by direct-to-LDS loads of whole 16-byte row chunks (chunks XOR-
    // swizzled by row; rows past N clamped to N - 1), and the fragments are
    // read from there after the prologue's barrier; otherwise each lane
    // loads its own row.
    bf16x8 qf[DC];
    unsigned char* qst = smem + (2 + NVB) * TILE + wave * 32 * RB;
    auto qdma = [&] {
#pragma unroll
        for (int j = 0; j < 32 * CPR / 64; ++j) {
            const int i = j * 64 + lane;
            const int row = i / CPR, pc = i % CPR;
            const int grow = min(qw + row, N - 1);
            __builtin_amdgcn_global_load_lds(Qg + (size_t)grow * rs + ((pc ^ (row & (CPR - 1))) << 3),
                                             (lds_void_t*)(qst + j * 1024), 16, 0, 0);
        }
    };
    if constexpr (QLDS) {
        qdma();
    } else {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (myq < N) v = ld16(Qg + (size_t)myq * rs + c * 16 + hi * 8);
            v ^= a.qsign;
            qf[c] = as_bf16x8(v);
        }
    }

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    // Row swizzles of the 16-byte chunks. K rows are read 16 rows at a time at
    // one chunk column; V rows are read by the transposing loads 4 rows x 64
    // bytes at a time.
    auto swk = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
    auto swv = [](int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };

    // Direct-to-LDS tile load: wave load j covers rows inst*RPI .. +RPI-1 of
    // the tile; lane i writes LDS chunk slot i, so it fetches the global chunk
    // that the swizzle puts there. Rows past N are clamped to N-1 (they are
    // masked for K and meet P = 0 for V).
    // Element offsets of this lane's chunks within a tile (row * rskv +
    // chunk) are fixed; a whole tile adds a uniform t * BN * rskv. Only the ragged
    // last tile recomputes them with the clamp.
    // The swizzle bits of a row depend only on the row's position within its
    // group of 16 (d = 128) or 8 row pairs (d = 64), and wave load j + 1
    // covers the rows of load j shifted by NW * RPI (a multiple of that
    // group), so one per-lane offset per tensor serves every load of the
    // tile; load j adds the uniform j * NW * RPI rows.
    static_assert((NL * RPI) % 16 == 0, "wave loads must keep the row swizzle");
    unsigned koff0, voff0;
    {
        const int row = wave * RPI + lane / CPR;
        const int slot = lane % CPR;
        koff0 = (unsigned)row * (unsigned)rskv + 8u * (unsigned)(slot ^ swk(row));
        voff0 = (unsigned)row * (unsigned)rskv + 8u * (unsigned)(slot ^ swv(row));
    }
    // Whole tiles load through buffer resources over this head's K and V rows:
    // the lane's byte offset is fixed and tile t, load j add the uniform
    // (t * BN + j * NW * RPI) row offset in an SGPR. A batch's rows span less
    // than 2^32 bytes (N * H * d < 2^31 elements), so every offset fits.
    const uint32_t span = (uint32_t)(((size_t)(N - 1) * rskv + D) * 2);   // bytes of this head's rows
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kg, span), vrs = buffer_rsrc(Vg, span);
    const uint32_t koffb = koff0 * 2u, voffb = voff0 * 2u;
    const uint32_t tile_b = (uint32_t)BN * (uint32_t)rskv * 2u;          // bytes per tile of rows
    const uint32_t jstep_b = (uint32_t)(NL * RPI) * (uint32_t)rskv * 2u;  // bytes between load j and j + 1
    // (The 4-wave d = 128 form keeps 64-bit per-lane addresses: measured 2-4%
    // faster there with them.)
    constexpr bool BUFLOAD = !(D == 128 && NW == 4);
    auto dma = [&](const __bf16* g, int t, int buf, bool is_v) {
        if (BUFLOAD && (t + 1) * BN <= N) {
            const uint32_t so = (uint32_t)t * tile_b;
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                const int inst = wave + NL * j;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? vrs : krs,
                                                         (lds_void_t*)(smem + buf * TILE + inst * 1024), 16,
                                                         is_v ? voffb : koffb, so + j * jstep_b, 0, 0);
            }
        } else if ((t + 1) * BN <= N) {
            const __bf16* gt = g + (size_t)t * BN * rskv;
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                const int inst = wave + NL * j;
                __builtin_amdgcn_global_load_lds(gt + j * (size_t)(NL * RPI) * rskv + (size_t)(is_v ? voff0 : koff0),
                                                 (lds_void_t*)(smem + buf * TILE + inst * 1024), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                const int inst = wave + NL * j;
                const int row = inst * RPI + lane / CPR;
                const int slot = lane % CPR;
                const int c = slot ^ (is_v ? swv(row) : swk(row));
                const int grow = min(t * BN + row, N - 1);
                __builtin_amdgcn_global_load_lds(g + (size_t)grow * rskv + c * 8,
                                                 (lds_void_t*)(smem + buf * TILE + inst * 1024), 16, 0, 0);
            }
        }
    };
    auto kbuf = [&](int i) { return smem + i * TILE; };
    auto vbuf = [&](int i) { return smem + (2 + i) * TILE; };
    // The loads of step t, issued as it starts: K_{t+2} and V_{t+1}.
    auto issue = [&](int t) {
        if (t + 2 < ntiles) dma(Kg, t + 2, t & 1, false);
        if (t + 1 < ntiles) dma(Vg, t + 1, 2 + (t + 1) % NVB, true);
    };
    const bool lag = PP && wave >= 4;     // a lagging wave (ping-pong)

    // Per-lane byte offsets of the MFMA operand reads. The swizzle only flips
    // address bits that the row base leaves clear, so the offset of d chunk cc
    // (K) or d block db (V) is the lane's base XOR a constant.
    int kbase;
    {
        const int sw = swk(l32);
        kbase = l32 * RB + ((hi ^ (sw & 1)) << 4) + ((sw >> 1) << 5);   // chunk pair cc: ^ (cc << 5)
    }
    int vbase;
    {
        const int g = lane >> 4, i = lane & 15;
        const int e = i >> 2;                              // key within the group of 4
        const int x = 2 * (g & 1) + ((i & 3) >> 1);        // chunk within the 64-byte run
        const int sq = (D == 128 ? e : (e >> 1));          // swizzle of that key row, in quads
        vbase = (4 * hi + e) * RB + (sq << 6) + (x << 4) + ((i & 1) << 3);   // d block db: ^ (db << 6)
    }

    auto wait_dma = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
    int vhi[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        vhi[db] = (vbase ^ (db << 6)) + 2 * TILE;
        if constexpr (PP) pin_vgpr(vhi[db]);
    }

    auto scores = [&](f32x16 (&s)[KB], const unsigned char* Ks) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + kb * 32 * RB + (kbase ^ (cc << 5)));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[cc], s[kb], 0, 0, 0);
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m = -INFINITY;   // reference max of S * c2 (base-2 units) for query myq
    float l = 0.f;         // running sum over this lane's keys (other half added at the end)
    const float c2 = a.c2;

    // Masking (tiles straddling the causal diagonal or the ragged end only:
    // masked scores become -inf; c2 > 0, so their exponentials are exactly
    // 0), row maximum and the lazy rescale of l and O for tile t in s.
    auto apply_mask = [&](int t, f32x16 (&s)[KB], auto masked_c) {
        if constexpr (decltype(masked_c)::value) {
            // Key of element u of block kb is j0 + kb*32 + 4*hi + 8*(u/4) + u%4.
            const int lim = CAUSAL ? min(N - 1, myq) : N - 1;   // last visible key
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int thr = lim - (t * BN + kb * 32 + 4 * hi);
#pragma unroll
                for (int u = 0; u < 16; ++u) s[kb][u] = (8 * (u >> 2) + (u & 3) > thr) ? -INFINITY : s[kb][u];
            }
        }
    };
    auto rescale_to_max = [&](f32x16 (&s)[KB]) {
        // Four independent max chains instead of one serial chain.
        float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int u = 0; u < 16; u += 2)
                mc[(u / 2) % 4] = __builtin_fmaxf(__builtin_fmaxf(mc[(u / 2) % 4], s[kb][u]), s[kb][u + 1]);
        float mx = __builtin_fmaxf(__builtin_fmaxf(mc[0], mc[1]), __builtin_fmaxf(mc[2], mc[3]));
        mx = max_halves(mx);
        const float mt = mx * c2;   // -inf when every key of the row is masked in this tile
        if (__builtin_amdgcn_ballot_w64(mt > m + kTau) != 0) {
            const float mnew = __builtin_fmaxf(m, mt);
            const float alpha = exp2_fast(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
    };
    auto prepare = [&](int t, f32x16 (&s)[KB], auto masked_c) {
        apply_mask(t, s, masked_c);
        rescale_to_max(s);
    };

    // One pipeline step, scheduled by hand (sched_barrier fences keep the
    // order): while K_{t+2} and V_{t+1} stream into LDS, the 16 score MFMAs of
    // tile t+1 are interleaved with the exponentials of tile t (phase A, run
    // at raised wave priority so that the VALU-heavy phase of one wave is
    // not starved by the other wave's PV MFMAs), then the PV MFMAs of tile t
    // run (phase B). Between two barriers a leading wave runs A(t) then B(t)
    // and, in the ping-pong form, a lagging one B(t-1) then A(t): its barrier
    // falls between its A and B. In that interval the leading waves read V_t,
    // the lagging ones V_{t-1}, and V_{t+1} arrives; the leading waves issue
    // the interval's loads and wait for them before its closing barrier. K operands are read in batches of KBS MFMAs one batch
    // ahead (while a direct-to-LDS load is in flight the compiler can only
    // wait for all outstanding LDS reads, so reads issued one MFMA ahead
    // would be waited for at once); V operands PFV MFMAs ahead. For the last
    // tile the scores of a tile past the end are computed from stale LDS and
    // never used.
    constexpr int NS = KB * DC;           // score MFMAs per tile
    constexpr int NP = DB * (BN / 16);    // PV MFMAs per tile
    constexpr int KBS = 2;
    constexpr int PFV = 2;
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // In the ping-pong form R = t % U is known at compile time; otherwise the
    // buffer slots follow t at run time.
    auto step = [&](int t, f32x16 (&scur)[KB], f32x16 (&snext)[KB], auto masked_c, auto r_c) {
        constexpr int R = decltype(r_c)::value;
        if (!lag) issue(t);
        // Phase A. Score MFMA i: block i % KB, d chunk i / KB (two chains).
        // K operands are read in batches of KBS MFMAs, one batch ahead; the
        // first batch is in flight during prepare.
        const unsigned char* Ks = kbuf(PP ? (R + 1) & 1 : (t + 1) & 1);
        auto kread = [&](int i) {
            return *reinterpret_cast<const bf16x8*>(Ks + (i % KB) * 32 * RB + (kbase ^ ((i / KB) << 5)));
        };
        bf16x8 kfr[NS];
#pragma unroll
        for (int i = 0; i < KBS; ++i) kfr[i] = kread(i);
        fence();
        // The 8-wave form defers the tile maximum to the rare rescale path
        // (kSumLimit); the others have no registers for that path and take
        // the maximum first.
        if constexpr (PP)
            apply_mask(t, scur, masked_c);
        else
            prepare(t, scur, masked_c);
        fence();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) snext[kb] = f32x16{};
        // Two partial row sums; each partial is pinned in place after its add
        // so that the adds stay spread over phase A instead of being sunk to
        // the end of the step as one serial chain.
        float rsum[2] = {0.f, 0.f};
        u32x4 w[BN / 16];
        bf16x8 pb[BN / 16];
        // The exponentials of tile t run as a three-stage pipeline over the
        // score MFMAs, so that no slot waits on a result produced in the same
        // slot: pair q (elements 2q, 2q+1 flat over blocks) gets its fma two
        // slots ahead, its exp2 one slot ahead and its sum / bf16 pack in
        // slot q / PPS.
        constexpr int NPAIR = KB * 8;
        constexpr int PPS = NPAIR / NS;       // pairs per score MFMA
        static_assert(PPS * NS == NPAIR && PPS >= 1, "pairs must split evenly over the MFMAs");
        float x[NPAIR][2], e[NPAIR][2];
        auto valu_slot = [&](int i) {
#pragma unroll
            for (int q = (i + 2) * PPS; q < (i + 3) * PPS; ++q) {
                if (q < 0 || q >= NPAIR) continue;
                const int f = 2 * q, kb = f / 16, u = f % 16;
                x[q][0] = __builtin_fmaf(scur[kb][u], c2, -m);
                x[q][1] = __builtin_fmaf(scur[kb][u + 1], c2, -m);
            }
#pragma unroll
            for (int q = (i + 1) * PPS; q < (i + 2) * PPS; ++q) {
                if (q < 0 || q >= NPAIR) continue;
                e[q][0] = exp2_fast(x[q][0]);
                e[q][1] = exp2_fast(x[q][1]);
                pin_vgpr(e[q][0]);
                pin_vgpr(e[q][1]);
            }
#pragma unroll
            for (int q = i * PPS; q < (i + 1) * PPS; ++q) {
                if (q < 0 || q >= NPAIR) continue;
                const int f = 2 * q;
                rsum[q % 2] += e[q][0] + e[q][1];
                pin_vgpr(rsum[q % 2]);
                uint32_t pw = pack_bf16x2(e[q][0], e[q][1]);
                // Keeps the pack in phase A (not sunk past a lagging wave's
                // barrier into phase B).
                if constexpr (PP) pin_vgpr(pw);
                w[f / 8][(f % 8) / 2] = pw;
                if (f % 8 == 6) pb[f / 8] = as_bf16x8(w[f / 8]);
            }
        };
        __builtin_amdgcn_s_setprio(1);
        valu_slot(-2);
        fence();
        valu_slot(-1);
        fence();
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            snext[i % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[i], qf[i / KB], snext[i % KB], 0, 0, 0);
            fence();
            if (i % KBS == 0) {
#pragma unroll
                for (int r = i + KBS; r < i + 2 * KBS && r < NS; ++r) kfr[r] = kread(r);
            }
            valu_slot(i);
            fence();
        }
        float tsum = rsum[0] + rsum[1];
        if (PP && __builtin_amdgcn_ballot_w64(!(tsum <= kSumLimit)) != 0) {
            // Rare: somewhere in the wave this tile's maximum exceeds the
            // running one by more than log2(kSumLimit / 32).
            f32x16 sr[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sr[kb] = f32x16{};
                const int krow = min(t * BN + kb * 32 + l32, N - 1);   // rows past N are masked
#pragma unroll
                for (int cc = 0; cc < DC; ++cc) {
                    // One operand at a time: this path is rare, its registers are not.
                    const bf16x8 kf = as_bf16x8(ld16(Kg + (size_t)krow * rskv + cc * 16 + hi * 8));
                    sr[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[cc], sr[kb], 0, 0, 0);
                    fence();
                }
            }
            apply_mask(t, sr, masked_c);
            rescale_to_max(sr);
            fence();
            tsum = 0.f;
#pragma unroll
            for (int q = 0; q < NPAIR; ++q) {
                const int f = 2 * q, kb = f / 16, u = f % 16;
                const float e0 = exp2_fast(__builtin_fmaf(sr[kb][u], c2, -m));
                const float e1 = exp2_fast(__builtin_fmaf(sr[kb][u + 1], c2, -m));
                tsum += e0 + e1;
                w[f / 8][(f % 8) / 2] = pack_bf16x2(e0, e1);
                if (f % 8 == 6) pb[f / 8] = as_bf16x8(w[f / 8]);
                fence();
            }
        }
        l += tsum;
        if (lag) {
            // A lagging wave's barrier: phase A of tile t is done, phase B
            // follows in the next interval.
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        }

        // Phase B. PV MFMA j: key chunk j / DB, d block j % DB.
        // Above 64 KB of LDS (the upper V buffers of the ping-pong form) a
        // buffer's offset no longer fits a read's immediate offset: there the
        // reads start from the pinned per-d-block bases vhi (V region
        // included) and only the slot and chunk offsets stay immediate.
        const unsigned char* Vs = PP ? smem + (R % NVB) * TILE : vbuf(t & 1);
        auto vread = [&](int j) {
            const int kc = j / DB, db = j % DB;
            const int voff = (PP ? vhi[db] : (vbase ^ (db << 6))) + kc * 16 * RB;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Vs + voff));
            const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Vs + voff + 8 * RB));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vfr[NP];
#pragma unroll
        for (int j = 0; j < PFV; ++j) vfr[j] = vread(j);
        fence();
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[j], pb[j / DB], oacc[j % DB], 0, 0, 0);
            if (j + PFV < NP) vfr[j + PFV] = vread(j + PFV);
            fence();
        }
        if (!lag) {
            wait_dma();
            __syncthreads();
        }
    };

    // Prologue: K_0, V_0, K_1 into LDS, then S_0.
    if (!lag) {
        dma(Kg, 0, 0, false);
        dma(Vg, 0, 2, true);
        if (ntiles > 1) dma(Kg, 1, 1, false);
    }
    wait_dma();
    __syncthreads();
    if constexpr (QLDS) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            u32x4 v = *reinterpret_cast<const u32x4*>(qst + l32 * RB + (((2 * c + hi) ^ (l32 & (CPR - 1))) << 4));
            if (myq >= N) v = u32x4{0u, 0u, 0u, 0u};
            v ^= a.qsign;
            qf[c] = as_bf16x8(v);
        }
    }
    f32x16 sa[KB], sb[KB];
    scores(sa, kbuf(0));
    __syncthreads();   // Kbuf[0] receives K_2 in step 0

    // Tiles before t_split need no mask for any wave (they end before the
    // workgroup's first query and before N); the rest run the masked variant.
    // Causal waves whose rows all precede a tile run it fully masked (p = 0).
    const int t_split = min(CAUSAL ? q0 / BN : ntiles, (N % BN) ? ntiles - 1 : ntiles);
    // The running maximum starts at the first tile's (every row sees key 0).
    if constexpr (PP) {
        if (t_split > 0)
            prepare(0, sa, std::false_type{});
        else
            prepare(0, sa, std::true_type{});
    }

    // Step t runs with S_t in sa when t is even, in sb when odd.
    auto run = [&](int t, auto r_c, auto masked_c) {
        if constexpr (decltype(r_c)::value & 1)
            step(t, sb, sa, masked_c, r_c);
        else
            step(t, sa, sb, masked_c, r_c);
    };
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    using R3 = std::integral_constant<int, 3>;
    // Under the causal mask a wave stops computing at the first tile whose
    // keys all follow its last query (that tile and every later one give
    // p = 0), but keeps issuing its share of the loads and passing the
    // barriers until the workgroup is done.
    auto idle = [&](int tt) { return CAUSAL && tt * BN > qw + 31; };
    if constexpr (!PP) {
        int t = 0;
        for (; t + 1 < t_split; t += 2) {
            step(t, sa, sb, std::false_type{}, R0{});
            step(t + 1, sb, sa, std::false_type{}, R0{});
        }
        if (t < t_split) {
            step(t, sa, sb, std::false_type{}, R0{});
            ++t;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sa[kb] = sb[kb];
        }
        for (; t < ntiles; t += 2) {
            if (idle(t)) break;
            step(t, sa, sb, std::true_type{}, R0{});
            if (t + 1 < ntiles) {
                if (idle(t + 1)) {
                    ++t;
                    break;
                }
                step(t + 1, sb, sa, std::true_type{}, R0{});
            }
        }
        for (; t < ntiles; ++t) {
            issue(t);
            wait_dma();
            __syncthreads();
        }
    } else {
        // The unmasked steps run in whole unrolled bodies; the up to U - 1 that
        // remain join the masked ones (on a tile with nothing to mask the mask
        // changes no score).
        const int t_un = t_split - t_split % U;
        int t = 0;
        for (; t < t_un; t += U) {
            run(t, R0{}, std::false_type{});
            run(t + 1, R1{}, std::false_type{});
            if constexpr (U == 4) {
                run(t + 2, R2{}, std::false_type{});
                run(t + 3, R3{}, std::false_type{});
            }
        }
        // Masked steps, from a multiple of U; on leaving, t is the first step
        // not run.
        auto masked = [&](int tt, auto r_c) {
            if (tt >= ntiles || idle(tt)) return false;
            run(tt, r_c, std::true_type{});
            return true;
        };
        for (; t < ntiles; t += U) {
            if (!masked(t, R0{})) break;
            if (!masked(t + 1, R1{})) {
                t += 1;
                break;
            }
            if constexpr (U == 4) {
                if (!masked(t + 2, R2{})) {
                    t += 2;
                    break;
                }
                if (!masked(t + 3, R3{})) {
                    t += 3;
                    break;
                }
            }
        }
        for (; t < ntiles; ++t) {
            if (!lag) issue(t);
            wait_dma();
            __syncthreads();
        }
        // The lagging waves run B of their last tile after the last barrier.
        __syncthreads();
    }

    // Epilogue: O = O^T / l (rounded to bf16), LSE = ln-domain m + ln l.
    // O leaves through LDS: each wave stages its 32 rows in its own part of
    // the K/V buffers (idle since the last barrier), 16-byte chunks of a row
    // XOR-swizzled by the row, then writes whole 16-byte chunks of rows, so
    // that the global stores cover contiguous rows instead of 8 bytes of 32
    // rows per instruction.
    const float lt = sum_halves(l);
    const float inv = 1.0f / lt;
    static_assert(NW * 32 * RB <= (2 + NVB) * TILE, "O staging fits the K/V buffers");
    unsigned char* ow = smem + wave * 32 * RB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
            w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
            // Elements d0 .. d0 + 3, d0 = db*32 + 8g + 4hi: chunk db*4 + g, bytes 8hi .. 8hi + 7.
            *reinterpret_cast<u32x2*>(ow + l32 * RB + (((db * 4 + g) ^ (l32 & (CPR - 1))) << 4) + 8 * hi) = w;
        }
    }
#pragma unroll
    for (int j = 0; j < 32 * CPR / 64; ++j) {
        const int i = j * 64 + lane;
        const int row = i / CPR, ch = i % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ow + row * RB + ((ch ^ (row & (CPR - 1))) << 4));
        if (qw + row < N) st16(Og + (size_t)(qw + row) * rs + ch * 8, v);
    }
    if (myq < N && hi == 0) a.lse[(size_t)bh * N + myq] = (m + __builtin_log2f(lt)) * kLn2;
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const long long grid8 = (long long)((a.N + 255) / 256) * a.B * a.H;
    const bool eight = D == 128 ? a.N > kFwdShortN : (a.N >= kFwdShortN64 && grid8 >= kFwdMinWgs8);
    if (eight) {
        hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 8>), dim3((unsigned)grid8), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    const long long grid = (long long)((a.N + 127) / 128) * a.B * a.H;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
