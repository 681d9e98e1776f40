/*
 * fa_mi355x.h -- C ABI of libfa_mi355x: exact tiled softmax attention
 * (forward and backward) for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * What is computed. Exact softmax attention, per batch b and head h,
 *
 *     O = softmax(scale * Q K^T + causal mask) V,    LSE_i = ln sum_j exp(S_ij)
 *
 * tile by tile with an online softmax: the kernels keep a running row
 * maximum and row sum and rescale the partial output, so the N x N score and
 * probability matrices never reach device memory. Sources, cited by page
 * title and section:
 *   - "FlashAttention-2: atención eficiente en GPU para contextos largos",
 *     section "El coste de mover datos en secuencias largas": the
 *     conventional computation writes the full score and probability
 *     matrices to high-bandwidth memory, which is the cost avoided here;
 *   - same page, section "Bloques pequeños, normalización global": blocks are
 *     processed in fast on-chip memory and the online softmax rescales the
 *     running statistics and partial outputs; results equal exact attention
 *     up to floating-point ordering, and outputs and gradients are compared
 *     within a tolerance, not bit for bit;
 *   - same page, section "Tres mejoras en la utilización de la GPU": work is
 *     split over the sequence as well as batch and heads, query rows are
 *     split across wavefronts that share the K and V tiles, and non-matrix
 *     work (rescaling, boundary and causal-mask handling) is kept out of the
 *     inner loop;
 *   - "读懂FlashAttention-2：让长上下文注意力更高效地运行在GPU上", section
 *     "分块处理仍需保持全局归一化": the method is exact attention, not a sparse
 *     approximation.
 * The pages do not describe the backward algorithm; attn_bwd computes the
 * textbook gradients of the definition above (see attn_bwd).
 *
 * Conventions shared by every entry point.
 *   Layout   q, k, v, o, dO, dq, dk, dv are contiguous [B, N, H, d] tensors,
 *            d fastest (element (b, n, h, c) at ((b*N + n)*H + h)*d + c).
 *            lse is a contiguous fp32 [B, H, N] tensor, natural log.
 *   Types    attn_fwd / attn_bwd take raw bfloat16 bits (2 bytes per
 *            element); attn_fwd_fp32 takes IEEE fp32. Accumulation and all
 *            softmax statistics are fp32.
 *   Causal   causal != 0 masks key j for query i when j > i (query and key
 *            sequences have the same length N).
 *   Scale    any finite float; it multiplies Q K^T before masking.
 *   Sizes    B, H, N >= 1; d in {64, 128}; N * H * d < 2^31 and
 *            B * N * H * d < 2^40.
 *   Pointers device pointers (hipMalloc'd or equivalent), 16-byte aligned.
 *   Memory   the caller owns and allocates every buffer, workspace included,
 *            and the stream. The library never allocates, frees or
 *            synchronises. Inputs are read-only; outputs are fully
 *            overwritten and must not alias any input.
 *   Stream   work is enqueued on `stream` (NULL = the null stream) and the
 *            call returns without waiting. Faults inside a kernel surface at
 *            the caller's next synchronisation on that stream.
 *   Errors   every argument is validated before any HIP call, so a rejected
 *            call has no side effect. NaN or Inf inside the tensors are not
 *            checked and propagate.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued entry point. */
enum fa_status {
    FA_OK = 0,               /* work enqueued */
    FA_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, size <= 0 or too large, non-finite scale,
                                H not a multiple of Hkv */
    FA_ERR_UNSUPPORTED = 2,  /* head dimension d not in {64, 128} */
    FA_ERR_WORKSPACE = 3,    /* workspace null or smaller than attn_bwd_workspace_size() */
    FA_ERR_HIP = 4           /* a HIP launch reported an error (hipGetLastError) */
};

/*
 * attn_fwd -- bf16 forward of exact attention (definition above).
 *   q, k, v  [B, N, H, d] bf16 inputs.
 *   o        [B, N, H, d] bf16 output, rounded to nearest even from fp32.
 *   lse      [B, H, N] fp32 output: natural-log log-sum-exp of row i of the
 *            scaled, masked scores (the statistic attn_bwd consumes).
 * The online softmax runs in fp32 (base-2 internally); the probabilities fed
 * to the second product are rounded to bf16, the row sum uses them unrounded.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_fp32 -- the same forward with fp32 inputs, outputs and products
 * (no value is rounded below fp32). Arguments as for attn_fwd.
 */
int attn_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                  int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd needs for this
 * shape: two fp32 arrays [B, H, Npad] with Npad = 64 * ceil(N / 64), the row
 * statistics -D_i (D_i = dO_i . O_i) and LSE_i * log2(e), rounded up to 256
 * bytes.
 * Returns 0 for arguments attn_bwd would reject.
 */
size_t attn_bwd_workspace_size(int B, int H, int N, int d, int causal);

/*
 * attn_bwd -- bf16 gradients of exact attention with respect to q, k, v.
 *   q, k, v  forward inputs, [B, N, H, d] bf16.
 *   o, lse   the forward's outputs for these inputs (from attn_fwd).
 *   dO       upstream gradient dL/dO, [B, N, H, d] bf16.
 *   dq,dk,dv outputs, [B, N, H, d] bf16 (rounded to nearest even from fp32).
 *   workspace, workspace_bytes: caller-owned device scratch of at least
 *            attn_bwd_workspace_size(B, H, N, d, causal) bytes, 256-byte
 *            aligned; its contents on entry are ignored and on return are
 *            unspecified.
 * Gradients (chain rule through the row softmax; P is recomputed from q, k
 * and lse, never stored):
 *     D_i = dO_i . O_i,  dP = dO V^T,  dS = P o (dP - D),
 *     dV = P^T dO,  dQ = scale * dS K,  dK = scale * dS^T Q.
 * The result is deterministic: no atomics; repeated calls give identical bits.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * Grouped-query and multi-query attention (page "FlashAttention-T:
 * Optimización GPU para LLMs Escalables", section "Innovaciones técnicas
 * frente a FlashAttention original", which lists both as natively supported):
 * K and V have Hkv heads, H is a multiple of Hkv, and query head h attends
 * with K/V head h / (H / Hkv) (Hkv = 1 is multi-query attention, Hkv = H is
 * attn_fwd / attn_bwd).
 *
 * attn_fwd_gqa -- as attn_fwd, with k, v [B, N, Hkv, d] bf16; q, o
 *   [B, N, H, d]; lse [B, H, N].
 * attn_bwd_gqa -- as attn_bwd, with k, v, dk, dv [B, N, Hkv, d]: the gradient
 *   of a K/V head is the sum over the H / Hkv query heads that read it, in
 *   fp32. The workspace must hold at least attn_bwd_workspace_size(B, H, N,
 *   d, causal) bytes (sized by the query heads); then one workgroup sums all
 *   H / Hkv heads. Given attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, causal)
 *   bytes, it may instead split the heads of a K/V head over S workgroups
 *   that write fp32 partial dK, dV into the workspace, summed afterwards in a
 *   fixed order (a shape with few K/V heads, above all under the causal mask,
 *   otherwise leaves most of the chip idle). Either way the result is
 *   deterministic; the two ways may differ in the last bit of dK, dV.
 * attn_bwd_gqa_workspace_size -- bytes of workspace for the split form above
 *   (equal to attn_bwd_workspace_size when this shape is not split); 0 for
 *   arguments attn_bwd_gqa would reject.
 * Errors as for attn_fwd / attn_bwd, plus FA_ERR_INVALID_ARG when Hkv <= 0 or
 * H is not a multiple of Hkv.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int N, int d, int causal, float scale, hipStream_t stream);
int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int Hkv, int N, int d, int causal, float scale, hipStream_t stream);
size_t attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d, int causal);

/*
 * The stages of the backward, exported so that a caller can time or schedule
 * them separately. attn_bwd is exactly attn_bwd_dq_prep, then attn_bwd_dkdv,
 * on one stream and one workspace. attn_bwd_prep followed by attn_bwd_dq is
 * the same first stage in two launches: it leaves bitwise the same workspace
 * and dq (the fused kernel sums D_i in the same order).
 *
 * attn_bwd_prep -- fills the workspace: -D_i, where D_i = sum_c dO[b, i, h, c] *
 *   O[b, i, h, c] (the row statistic sum_j P_ij dP_ij of the softmax
 *   backward), then LSE_i * log2(e), fp32, with D = 0 and LSE = +inf on the
 *   padded rows.
 * attn_bwd_dkdv -- dk = scale * dS^T Q and dv = P^T dO: one workgroup per
 *   block of 128 keys, looping over query tiles; reads the workspace.
 * attn_bwd_dq -- dq = scale * dS K: one workgroup per block of 256 queries
 *   (128 for d = 64 or N <= 2048), looping over key tiles (recomputes P and
 *   dP); reads the workspace.
 * attn_bwd_dq_prep -- attn_bwd_dq that also does attn_bwd_prep's work: each
 *   lane forms -D and LSE * log2(e) of its own query from the dO row it holds
 *   and the O row, uses them, and writes them into the workspace for
 *   attn_bwd_dkdv. o and lse as for attn_bwd (FA_ERR_INVALID_ARG if null).
 * Arguments and errors as for attn_bwd.
 */
int attn_bwd_prep(const void* o, const void* dO, const float* lse, void* workspace, size_t workspace_bytes,
                  int B, int H, int N, int d, hipStream_t stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                  size_t workspace_bytes, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                  hipStream_t stream);
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                size_t workspace_bytes, void* dq, int B, int H, int N, int d, int causal, float scale,
                hipStream_t stream);
int attn_bwd_dq_prep(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* workspace, size_t workspace_bytes, void* dq,
                     int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_fp8 -- FP8 (OCP E4M3) forward (page "FlashAttention-T: Optimización
 * GPU para LLMs Escalables", section "Innovaciones técnicas frente a
 * FlashAttention original", which names 8-bit quantisation as supported):
 *   q8, k8   E4M3 bytes, [B, N, H, d], device, read-only.
 *   vt8      V transposed per head, E4M3 bytes, [B, H, d, ldv]: row (b, h, c)
 *            holds V[b, :, h, c] for keys 0 .. N-1 contiguously; bytes N ..
 *            ldv-1 of each row are padding: read, but cleared before use, so
 *            they may hold anything (NaN codes included).
 *   ldv      bytes per vt8 row: a multiple of 16 and at least 64 * ceil(N/64).
 *   q_descale, k_descale, v_descale: per-tensor factors, finite and > 0; the
 *            real inputs are value * descale.
 *   o        output [B, N, H, d] bf16; lse output [B, H, N] fp32 (natural log).
 *   d        must be 128.
 * Scores S = scale * (q8 * q_descale)(k8 * k_descale)^T are exact products of
 * E4M3 values summed in fp32; the online softmax keeps the exact running
 * maximum over 64-key tiles, so P = exp(S - m) <= 1; P is rounded to E4M3
 * (nearest even) for the P V product while the row sum l and LSE use the
 * unrounded P; O = v_descale * (sum of rescaled E4M3(P) V8) / l.
 * Errors: as attn_fwd, plus FA_ERR_INVALID_ARG for a descale that is not
 * finite and positive or a bad ldv, and FA_ERR_UNSUPPORTED for d != 128.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, int ldv,
                 float q_descale, float k_descale, float v_descale, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * Decoding against a key/value cache (page "FlashAttention-2: atención
 * eficiente en GPU para contextos largos", section "Cómo documentar una
 * diferencia técnica", which separates the first pass over a context from
 * token-by-token generation). The same exact attention as attn_fwd_gqa for
 * Nq new query rows against Nk cached keys; query i is the token at position
 * Nk - Nq + i, so with causal != 0 it sees keys j <= Nk - Nq + i (the mask is
 * aligned to the last key; with Nq = Nk it is attn_fwd_gqa's).
 *
 * attn_decode_workspace_size -- bytes of scratch attn_decode needs for this
 *   shape (per-chunk partial outputs and LSE, fp32); 0 if the shape is
 *   rejected.
 * attn_decode -- bf16 decoding, split over the key range:
 *   q        [B, Nq, H, d] bf16, device, read-only.
 *   k, v     the cache, [B, Nk, Hkv, d] bf16 (d fastest), device, read-only.
 *   o        output [B, Nq, H, d] bf16, fully overwritten.
 *   lse      output [B, H, Nq] fp32, natural-log log-sum-exp of each row.
 *   workspace, workspace_bytes: caller-owned device scratch of at least
 *            attn_decode_workspace_size(...) bytes, 256-byte aligned; its
 *            contents on entry are ignored and on return are unspecified.
 *   B, H, Hkv, Nq, Nk, d: H a multiple of Hkv; d in {64, 128}.
 * Each chunk of keys gives every query row the attention restricted to it,
 *     O_s (normalised within the chunk) and LSE_s,
 * and the rows are combined exactly:
 *     LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
 * Errors: FA_ERR_INVALID_ARG for a null or unaligned pointer, B, H, Hkv, Nq
 * or Nk < 1, H not a multiple of Hkv, causal with Nq > Nk, a non-finite scale
 * or sizes past the limits of attn_fwd; FA_ERR_UNSUPPORTED for d not in
 * {64, 128} or more than 32 query rows per K/V head ((H / Hkv) * Nq > 32);
 * FA_ERR_WORKSPACE for a null, unaligned or too small workspace;
 * FA_ERR_HIP when a launch fails. Asynchronous on `stream`.
 */
size_t attn_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d);
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes,
                int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory (code recorded under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same backward, same kernels and
 * bitwise the same dq, dk, dv, with the workspace taken from a static device
 * array of FA_NOALLOC_SCRATCH_BYTES inside the library instead of from the
 * caller. The call allocates and frees nothing.
 *   Arguments as attn_bwd, without workspace and workspace_bytes; `stream`
 *   must belong to the current device (hipSetDevice).
 *   Limit: attn_bwd_workspace_size(B, H, N, d, causal) must not exceed
 *   FA_NOALLOC_SCRATCH_BYTES (16 MiB: B * H * 64 * ceil(N / 64) up to
 *   2,097,152 rows, e.g. 16 heads of 131072 tokens); larger shapes return
 *   FA_ERR_WORKSPACE before any HIP call.
 *   Sharing: each GPU holds one copy of the array until the process ends,
 *   and every call on that GPU uses it. Calls that overlap on one GPU (on
 *   different streams, or from several threads without ordering) race on
 *   it; order them on one stream or with events. Nothing in it needs
 *   clearing between calls.
 *   The first call on a device looks up the array's address there
 *   (hipGetSymbolAddress); FA_ERR_HIP if that fails.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/* fa_status_string -- static, human-readable name of a status code. Never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
