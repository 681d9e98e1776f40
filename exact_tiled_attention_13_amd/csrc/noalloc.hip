// noalloc.hip -- attn_bwd_noalloc: attn_bwd with its workspace in a static
// device array instead of caller memory (C ABI in include/fa_mi355x.h).
//
// The backward's workspace (the row statistics -D and LSE * log2(e), written
// by the first stage and read by the other two) lives in `scratch`, a
// file-scope device array of FA_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds until the process ends. Host code never passes
// `scratch` itself to a kernel (on the host it is only a stand-in symbol):
// the first call on a device looks up that device's copy with
// hipGetSymbolAddress, with the device current, and every later call on it
// reuses the address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa_mi355x.h"

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, looked up once per device.
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FA_OK;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                int causal, float scale, hipStream_t stream) {
    // Argument checks first, with no HIP call: attn_bwd validates everything before its workspace, so with
    // no workspace it returns the argument error of a bad call and FA_ERR_WORKSPACE for a good one.
    const int st = attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, nullptr, 0, B, H, N, d, causal, scale, stream);
    if (st != FA_ERR_WORKSPACE) return st == FA_OK ? FA_ERR_HIP : st;
    const size_t need = attn_bwd_workspace_size(B, H, N, d, causal);
    if (need == 0 || need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
    void* ws = nullptr;
    const int sst = scratch_of_current_device(&ws);
    if (sst != FA_OK) return sst;
    // The first stage overwrites every workspace byte the later stages read, so nothing needs clearing.
    return attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, ws, FA_NOALLOC_SCRATCH_BYTES, B, H, N, d, causal, scale,
                    stream);
}
