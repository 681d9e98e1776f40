/*
 * fa_micro.h -- C ABI of libfa_micro: microbenchmarks and probes of the
 * MI355X (gfx950) units that bound the attention kernels. They measure the
 * hardware, not the method: each one isolates the unit that one design
 * decision of the attention library rests on.
 *
 *   fa_micro_mfma_bf16   sustained rate of v_mfma_f32_32x32x16_bf16 (the
 *                        product both attention contractions run on) and
 *                        the shader clock the chip holds while running it;
 *   fa_micro_exp2        issue rate of v_exp_f32, the exponential of the
 *                        online softmax (one per score);
 *   fa_micro_fp8_dot     the fp32 sums that v_mfma_scale_f32_32x32x64_f8f6f4
 *                        forms from E4M3 products (their accumulation error
 *                        sets the FP8 forward's tolerance);
 *   fa_micro_atomic_add  throughput of coalesced fp32 global atomic adds (the
 *                        cost of accumulating dQ with atomics).
 *
 * Conventions: pointers are device pointers (hipMalloc'd or equivalent,
 * 16-byte aligned); every call validates its arguments before any HIP call,
 * enqueues on `stream` and returns without waiting; nothing is allocated.
 * Return values: 0 on success, 1 for an invalid argument, 4 when the launch
 * reported a HIP error (the fa_status codes of fa_mi355x.h).
 *
 * Clock stamps: kernels that take `clk` write, for each workgroup w, four
 * 64-bit words clk[4w .. 4w+3] = {shader-clock counter at start, at end,
 * 100 MHz real-time counter at start, at end}, read by the first lane of the
 * workgroup's first wave (s_memtime and s_memrealtime). The ratio of the two
 * counters' advances, times 100 MHz, is the shader clock over that interval.
 */
#ifndef FA_MICRO_H
#define FA_MICRO_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_micro_mfma_bf16 -- `blocks` workgroups of 256 threads; each wave issues
 * `iters` rounds of four v_mfma_f32_32x32x16_bf16 (32768 FLOP each) into
 * four independent accumulators. Operands by `mode`: 0 -- one constant
 * register pair (no operand bit ever changes); 1 -- eight register pairs of
 * pseudo-random values in [-2, 2) used in turn; 2 -- as 1, but the A operand
 * of every product is read from LDS (ds_read_b128 of pseudo-random values,
 * 1 KB per product per wave); 3 -- both operands read from LDS (2 KB per
 * product per wave: at one product per 32 clocks on all four SIMDs, 256
 * bytes per clock per CU); 4 and 5 -- as 1, with one and two accumulator
 * chains instead of four (each product depends on the one issued one or two
 * products earlier). The modes separate the energy of the matrix
 * cores' arithmetic from that of their operand traffic (the chip lowers its
 * clock as its power rises). out: blocks * 256 floats (one checksum per
 * thread, so that no product is dropped). clk: 4 * blocks words.
 * FLOP = blocks * 4 waves * iters * 4 * 32768. blocks >= 1, 2 <= iters <= 2^24,
 * iters even; mode in {0, ..., 5}.
 */
int fa_micro_mfma_bf16(float* out, unsigned long long* clk, int blocks, int iters, int mode, hipStream_t stream);

/*
 * fa_micro_mfma_valu -- whether a wave's own VALU work hides under its MFMAs:
 * `blocks` workgroups of 256 threads (launched for two waves per SIMD); each
 * wave runs `iters` rounds of four v_mfma_f32_32x32x16_bf16 (random register
 * operands, four chains), each followed by `nfma` independent v_fma_f32 and
 * `nexp` v_exp_f32. (nfma, nexp) in {(0,0), (2,0), (4,0), (8,0), (0,1),
 * (0,2), (0,4), (4,2), (6,2)}. out: blocks * 256 floats; clk: 4 * blocks
 * words. FLOP = blocks * 4 * iters * 4 * 32768.
 */
int fa_micro_mfma_valu(float* out, unsigned long long* clk, int blocks, int iters, int nfma, int nexp,
                       hipStream_t stream);

/*
 * fa_micro_exp2 -- `blocks` workgroups of 256 threads; each lane runs eight
 * independent chains x <- exp2(-x) for `iters` steps (one v_exp_f32 each).
 * out: blocks * 256 floats. clk: 4 * blocks words. Instructions per wave:
 * 8 * iters. blocks >= 1, 1 <= iters <= 2^24.
 */
int fa_micro_exp2(float* out, unsigned long long* clk, int blocks, int iters, hipStream_t stream);

/*
 * fa_micro_fp8_dot -- `problems` independent products C = sum_s A_s B_s on
 * the FP8 matrix cores, one 64-lane workgroup each, `chain` MFMAs per
 * problem (each adding a 32 x 64 by 64 x 32 product into the fp32
 * accumulator, which starts at zero):
 *   a  E4M3 bytes [problems][chain][32 rows][64], row-major;
 *   b  E4M3 bytes [problems][chain][32 columns][64]: column j's 64 bytes
 *      contiguous;
 *   c  fp32 [problems][32][32], row-major, written.
 * Both operands use format selector 0 (E4M3) and no block scales.
 * problems >= 1, 1 <= chain <= 64.
 */
int fa_micro_fp8_dot(const void* a, const void* b, float* c, int problems, int chain, hipStream_t stream);

/*
 * fa_micro_atomic_add -- n threads (n a multiple of 256); thread i adds
 * 1.0f to buf[i] `reps` times with a global atomic add (consecutive lanes,
 * consecutive words). Bytes moved = 4 * n * reps. n >= 256, reps >= 1.
 */
int fa_micro_atomic_add(float* buf, long long n, int reps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MICRO_H */
