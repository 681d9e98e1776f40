// kernels.hpp -- host-side launchers of the libfa_mi355x kernels (internal).
//
// Each launcher assumes its arguments were validated by the C-ABI layer
// (api.cpp): non-null aligned pointers, B, H, N >= 1, d in {64, 128}. It
// enqueues on `stream` and returns hipGetLastError() after the launch(es).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>

#include "common.hpp"

namespace fa {

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp32(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_prep(const BwdArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t stream);
// prep: the dQ kernel also computes the row statistics bwd_prep would (from
// a.o, a.dO, a.lse) and writes them to a.dd / a.lse2 for the dK/dV kernel.
hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, bool prep, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream);
// Split kernel over (chunk, K/V head, batch), then the merge over query rows.
hipError_t launch_decode(const DecodeArgs& a, int d, bool causal, hipStream_t stream);

// Key chunking of a decode call: S chunks of L keys (L a multiple of 32). The
// split kernel holds 48 KB of LDS per one-wave workgroup, so a CU runs three
// at a time and the chip 768; the chunks are sized so that the grid fills
// that exactly once (a partial second round measured up to 20% slower, two
// full rounds 7% slower than one; fewer chunks also shrink the merge). Grids
// with more than 768 (K/V head, batch) pairs get one chunk each. Used for both
// the launch and the workspace size, so the two always agree.
inline int decode_chunks(int B, int Hkv, int Nk, int* L) {
    constexpr long long kSlots = 256 * 3;   // CUs x split workgroups per CU
    const long long units = (long long)B * Hkv;
    const long long tiles = (Nk + 31) / 32;
    long long want = kSlots / units;
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const long long per = (Nk + want - 1) / want;
    const int l = (int)((per + 31) / 32 * 32);
    *L = l;
    return (int)((Nk + l - 1) / l);
}

// Grouped-query dK/dV: the number S of workgroups over which the G = H / Hkv
// query heads of one (key block, K/V head, batch) are divided (S divides G;
// each part writes fp32 partial sums that a reduction adds up). With few K/V
// heads the unsplit grid can be no larger than the chip, and under the causal
// mask its workgroups differ in length up to N / 128 times, so the first key
// block alone sets the time. Each candidate S is scored by simulating the
// dispatch: workgroup ids go round-robin to the 8 XCDs, xcd_remap gives each
// XCD a contiguous range of (part, key block) pairs, and an XCD starts its
// next workgroup on whichever of its slots (32 CUs x workgroups per CU) frees
// first; a workgroup costs its 64-query tiles times its heads (about 1.8 us
// per tile at d = 128, 1 us at d = 64), and a split adds its partial sums'
// HBM traffic at 4 TB/s. A larger S must win by 3%. Grids of at least four
// workgroups per slot are left unsplit.
inline int dkdv_gqa_splits_uncached(int B, int H, int Hkv, int N, int d, bool causal) {
    const int G = H / Hkv;
    if (G <= 1) return 1;
    const long long nk = (N + 127) / 128;
    const long long units = nk * B * Hkv;
    const int slots = d == 128 ? 32 : 64;
    if (units >= 4LL * 8 * slots) return 1;
    const double tile_us = d == 128 ? 1.8 : 1.0;
    const double elems = (double)B * N * Hkv * d;
    double best = -1.0;
    int best_s = 1;
    for (int S = 1; S <= G; ++S) {
        if (G % S != 0) continue;
        const long long total = units * S;
        if (total > 16384) break;
        const long long per = total / 8, rem = total % 8;
        long long span = 0;
        for (long long x = 0; x < 8; ++x) {
            const long long cnt = per + (x < rem ? 1 : 0);
            const long long start = x * per + std::min(x, rem);
            std::priority_queue<long long, std::vector<long long>, std::greater<long long>> free_at;
            for (int i = 0; i < slots; ++i) free_at.push(0);
            for (long long k = 0; k < cnt; ++k) {
                const long long kb = (start + k) % nk;
                const long long qstart = causal ? kb * 128 : 0;
                const long long cost = (N - qstart + 63) / 64 * (G / S);
                const long long t = free_at.top() + cost;
                free_at.pop();
                free_at.push(t);
                span = std::max(span, t);
            }
        }
        double us = (double)span * tile_us;
        if (S > 1) us += (2.0 * S * 2 * 4 * elems + 2 * 2 * elems) / 4e6;
        if (best < 0.0 || us < 0.97 * best) {
            best = us;
            best_s = S;
        }
    }
    return best_s;
}

// dkdv_gqa_splits_uncached memoised per shape: the simulation walks up to
// 16384 workgroups per candidate, which a caller repeating one shape (every
// training step) should not pay on each call. The table only grows with the
// number of distinct shapes a process uses; a mutex guards it.
inline int dkdv_gqa_splits(int B, int H, int Hkv, int N, int d, bool causal) {
    if (H / Hkv <= 1) return 1;
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int, int, bool>, int> memo;
    const auto key = std::make_tuple(B, H, Hkv, N, d, causal);
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = memo.find(key);
        if (it != memo.end()) return it->second;
    }
    const int s = dkdv_gqa_splits_uncached(B, H, Hkv, N, d, causal);
    std::lock_guard<std::mutex> lock(mu);
    memo.emplace(key, s);
    return s;
}

}  // namespace fa
