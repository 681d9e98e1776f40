// api.cpp -- the C ABI of libfa_mi355x (declared in include/fa_mi355x.h).
//
// Validates every argument before touching HIP, derives the kernel
// constants (base-2 softmax scale, sign folding) and calls the launchers.
// Nothing here allocates, frees or synchronises.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa_mi355x.h"
#include "kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int B, int H, int N, int d, float scale) {
    if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const long long per_batch = (long long)N * H * d;
    if (per_batch >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    if ((long long)B * per_batch >= (1LL << 40)) return FA_ERR_INVALID_ARG;
    // Grid sizes: (ceil(N/128) * B * H) workgroups must fit a 32-bit grid.
    if ((long long)((N + 127) / 128) * B * H >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

int check_heads(int H, int Hkv) {
    if (Hkv <= 0 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

void fill_scale(float scale, float& c2, uint32_t& qsign, float& qsign_f) {
    // c2 is kept at least FLT_MIN so that masked scores (-inf) times c2 stay
    // -inf; for |scale| that small every exponent rounds to exp2(0) anyway.
    c2 = fmaxf(fabsf(scale) * fa::kLog2e, FLT_MIN);
    const bool neg = signbit(scale) && scale != 0.0f;
    qsign = neg ? 0x80008000u : 0u;
    qsign_f = neg ? -1.0f : 1.0f;
}

// Backward workspace: D and LSE*log2(e), each fp32 [B, H, Npad], Npad = 64 * ceil(N / 64).
size_t ws_half_elems(int B, int H, int N) { return (size_t)B * H * (size_t)((N + 63) & ~63); }

size_t ws_bytes(int B, int H, int N) {
    const size_t raw = 2 * ws_half_elems(B, H, N) * sizeof(float);
    return (raw + 255) & ~(size_t)255;
}

int check_ws(const void* ws, size_t bytes, int B, int H, int N) {
    if (ws == nullptr || !aligned16(ws) || bytes < ws_bytes(B, H, N)) return FA_ERR_WORKSPACE;
    return FA_OK;
}

// Grouped-query backward: after the statistics, room for the fp32 partial
// dK, dV of a split dK/dV stage ([S][2][B, N, Hkv, d]).
size_t gqa_part_bytes(int B, int Hkv, int N, int d, int S) {
    if (S <= 1) return 0;
    const size_t raw = (size_t)S * 2 * (size_t)B * N * Hkv * d * sizeof(float);
    return (raw + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, hipStream_t stream) {
    int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    st = check_heads(H, Hkv);
    if (st != FA_OK) return st;
    st = check_ptrs({q, k, v, o, lse});
    if (st != FA_OK) return st;
    fa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.Hkv = Hkv;
    fill_scale(scale, a.c2, a.qsign, a.qsign_f);
    return fa::launch_fwd_bf16(a, d, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             int causal, float scale, hipStream_t stream) {
    return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, int ldv, float q_descale, float k_descale,
                 float v_descale, void* o, float* lse, int B, int H, int N, int d, int causal, float scale,
                 hipStream_t stream) {
    int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    const float descales[3] = {q_descale, k_descale, v_descale};
    for (float x : descales)
        if (!isfinite(x) || !(x > 0.0f)) return FA_ERR_INVALID_ARG;
    if (ldv < (N + 63) / 64 * 64 || ldv % 16 != 0) return FA_ERR_INVALID_ARG;
    if ((long long)B * H * d * (long long)ldv >= (1LL << 40)) return FA_ERR_INVALID_ARG;
    st = check_ptrs({q8, k8, vt8, o, lse});
    if (st != FA_OK) return st;
    fa::Fp8Args a{};
    a.q = q8; a.k = k8; a.vt = vt8; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.ldv = ldv;
    const float eff = scale * q_descale * k_descale;
    float unused_f;
    uint32_t unused_s;
    fill_scale(eff, a.c2, unused_s, unused_f);
    a.qsign = (signbit(eff) && eff != 0.0f) ? 0x80808080u : 0u;
    a.dv = v_descale;
    return fa::launch_fwd_fp8(a, d, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int attn_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                  int d, int causal, float scale, hipStream_t stream) {
    int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    st = check_ptrs({q, k, v, o, lse});
    if (st != FA_OK) return st;
    fa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.Hkv = H;
    fill_scale(scale, a.c2, a.qsign, a.qsign_f);
    return fa::launch_fwd_fp32(a, d, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t attn_bwd_workspace_size(int B, int H, int N, int d, int causal) {
    (void)causal;
    if (check_shape(B, H, N, d, 1.0f) != FA_OK) return 0;
    return ws_bytes(B, H, N);
}

int attn_bwd_prep(const void* o, const void* dO, const float* lse, void* workspace, size_t workspace_bytes, int B,
                  int H, int N, int d, hipStream_t stream) {
    int st = check_shape(B, H, N, d, 1.0f);
    if (st != FA_OK) return st;
    st = check_ptrs({o, dO, lse});
    if (st != FA_OK) return st;
    st = check_ws(workspace, workspace_bytes, B, H, N);
    if (st != FA_OK) return st;
    fa::BwdArgs a{};
    a.o = o; a.dO = dO; a.lse = lse;
    a.dd = static_cast<float*>(workspace);
    a.lse2 = a.dd + ws_half_elems(B, H, N);
    a.B = B; a.H = H; a.N = N; a.Hkv = H;
    return fa::launch_bwd_prep(a, d, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

int fill_bwd(fa::BwdArgs& a, const void* q, const void* k, const void* v, const void* dO, const void* workspace,
             size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale) {
    int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    st = check_heads(H, Hkv);
    if (st != FA_OK) return st;
    st = check_ptrs({q, k, v, dO});
    if (st != FA_OK) return st;
    st = check_ws(workspace, workspace_bytes, B, H, N);
    if (st != FA_OK) return st;
    a.q = q; a.k = k; a.v = v; a.dO = dO;
    a.dd = static_cast<float*>(const_cast<void*>(workspace));
    a.lse2 = a.dd + ws_half_elems(B, H, N);
    a.B = B; a.H = H; a.N = N; a.Hkv = Hkv;
    a.scale = scale;
    float unused;
    fill_scale(scale, a.c2, a.qsign, unused);
    return FA_OK;
}

int dkdv_stage(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
               size_t workspace_bytes, void* dk, void* dv, int B, int H, int Hkv, int N, int d, int causal,
               float scale, hipStream_t stream) {
    fa::BwdArgs a{};
    int st = fill_bwd(a, q, k, v, dO, workspace, workspace_bytes, B, H, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    st = check_ptrs({dk, dv});
    if (st != FA_OK) return st;
    a.dk = dk; a.dv = dv;
    // Split the query heads of a K/V head when the caller's workspace has
    // room for the partial sums (attn_bwd_gqa_workspace_size); else unsplit.
    a.gsplit = 1;
    if (Hkv != H) {
        const int S = fa::dkdv_gqa_splits(B, H, Hkv, N, d, causal != 0);
        const size_t base = ws_bytes(B, H, N);
        if (S > 1 && workspace_bytes >= base + gqa_part_bytes(B, Hkv, N, d, S)) {
            a.gsplit = S;
            a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(const_cast<void*>(workspace)) + base);
        }
    }
    return fa::launch_bwd_dkdv(a, d, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// o and lse non-null: the fused form that also fills the workspace's statistics.
int dq_stage(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             const void* workspace, size_t workspace_bytes, void* dq, int B, int H, int Hkv, int N, int d,
             int causal, float scale, hipStream_t stream) {
    fa::BwdArgs a{};
    int st = fill_bwd(a, q, k, v, dO, workspace, workspace_bytes, B, H, Hkv, N, d, scale);
    if (st != FA_OK) return st;
    const bool prep = o != nullptr || lse != nullptr;
    st = prep ? check_ptrs({dq, o, lse}) : check_ptrs({dq});
    if (st != FA_OK) return st;
    a.dq = dq;
    a.o = o;
    a.lse = lse;
    return fa::launch_bwd_dq(a, d, causal != 0, prep, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                  size_t workspace_bytes, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                  hipStream_t stream) {
    return dkdv_stage(q, k, v, dO, workspace, workspace_bytes, dk, dv, B, H, H, N, d, causal, scale, stream);
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                size_t workspace_bytes, void* dq, int B, int H, int N, int d, int causal, float scale,
                hipStream_t stream) {
    return dq_stage(q, k, v, nullptr, dO, nullptr, workspace, workspace_bytes, dq, B, H, H, N, d, causal, scale,
                    stream);
}

int attn_bwd_dq_prep(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     void* workspace, size_t workspace_bytes, void* dq, int B, int H, int N, int d, int causal,
                     float scale, hipStream_t stream) {
    if (o == nullptr || lse == nullptr) return FA_ERR_INVALID_ARG;
    return dq_stage(q, k, v, o, dO, lse, workspace, workspace_bytes, dq, B, H, H, N, d, causal, scale, stream);
}

size_t attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d, int causal) {
    if (check_shape(B, H, N, d, 1.0f) != FA_OK || check_heads(H, Hkv) != FA_OK) return 0;
    const int S = Hkv == H ? 1 : fa::dkdv_gqa_splits(B, H, Hkv, N, d, causal != 0);
    return ws_bytes(B, H, N) + gqa_part_bytes(B, Hkv, N, d, S);
}

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, hipStream_t stream) {
    int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    st = check_heads(H, Hkv);
    if (st != FA_OK) return st;
    st = check_ptrs({q, k, v, o, dO, lse, dq, dk, dv});
    if (st != FA_OK) return st;
    st = check_ws(workspace, workspace_bytes, B, H, N);
    if (st != FA_OK) return st;
    // dQ first: its kernel also writes the row statistics the dK/dV kernel reads.
    st = dq_stage(q, k, v, o, dO, lse, workspace, workspace_bytes, dq, B, H, Hkv, N, d, causal, scale, stream);
    if (st != FA_OK) return st;
    return dkdv_stage(q, k, v, dO, workspace, workspace_bytes, dk, dv, B, H, Hkv, N, d, causal, scale, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
             int causal, float scale, hipStream_t stream) {
    return attn_bwd_gqa(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d, causal, scale,
                        stream);
}

}  // extern "C"

namespace {

// Decode shape checks and workspace layout: per-chunk outputs fp32
// [B, Hkv, S, R, d], then per-chunk LSE fp32 [B, Hkv, S, R].
int check_decode(int B, int H, int Hkv, int Nq, int Nk, int d, float scale) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)Nk * Hkv * d >= (1LL << 31) || (long long)Nq * H * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    if ((long long)B * Nk * Hkv * d >= (1LL << 40)) return FA_ERR_INVALID_ARG;
    if ((long long)(H / Hkv) * Nq > 32) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

size_t decode_part_elems(int B, int H, int Hkv, int Nq, int Nk, int d) {
    int L;
    const int S = fa::decode_chunks(B, Hkv, Nk, &L);
    return (size_t)B * Hkv * S * (size_t)((H / Hkv) * Nq) * d;
}

size_t decode_ws_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
    const size_t o = decode_part_elems(B, H, Hkv, Nq, Nk, d);
    const size_t raw = (o + o / d) * sizeof(float);
    return (raw + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d) {
    if (check_decode(B, H, Hkv, Nq, Nk, d, 1.0f) != FA_OK) return 0;
    return decode_ws_bytes(B, H, Hkv, Nq, Nk, d);
}

int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                hipStream_t stream) {
    int st = check_decode(B, H, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
    st = check_ptrs({q, k, v, o, lse});
    if (st != FA_OK) return st;
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < decode_ws_bytes(B, H, Hkv, Nq, Nk, d))
        return FA_ERR_WORKSPACE;
    fa::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk;
    a.R = (H / Hkv) * Nq;
    a.S = fa::decode_chunks(B, Hkv, Nk, &a.L);
    a.opart = static_cast<float*>(workspace);
    a.lpart = a.opart + decode_part_elems(B, H, Hkv, Nq, Nk, d);
    float unused;
    fill_scale(scale, a.c2, a.qsign, unused);
    return fa::launch_decode(a, d, causal != 0, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: return "FA_ERR_UNKNOWN";
    }
}

}  // extern "C"
