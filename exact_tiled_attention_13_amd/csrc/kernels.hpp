// kernels.hpp -- host-side launchers of the libfa_mi355x kernels (internal).
//
// Each launcher assumes its arguments were validated by the C-ABI layer
// (api.cpp): non-null aligned pointers, B, H, N >= 1, d in {64, 128}. It
// enqueues on `stream` and returns hipGetLastError() after the launch(es).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fa {

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp32(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_prep(const BwdArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream);
// Split kernel over (chunk, K/V head, batch), then the merge over query rows.
hipError_t launch_decode(const DecodeArgs& a, int d, bool causal, hipStream_t stream);

// Key chunking of a decode call: S chunks of L keys (L a multiple of 32),
// about 2048 split workgroups in all. Used for both the launch and the
// workspace size, so the two always agree.
inline int decode_chunks(int B, int Hkv, int Nk, int* L) {
    const long long units = (long long)B * Hkv;
    const long long tiles = (Nk + 31) / 32;
    long long want = (2048 + units - 1) / units;
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const long long per = (Nk + want - 1) / want;
    const int l = (int)((per + 31) / 32 * 32);
    *L = l;
    return (int)((Nk + l - 1) / l);
}

}  // namespace fa
