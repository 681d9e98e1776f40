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

}  // namespace fa
