/*
 * moe_peaks.h — C ABI of libmoe_peaks.so: the two kernels that measure what
 * an MI355X actually sustains, so the MoE kernels' rates can be stated
 * against the measured ceilings as well as the published ones (8 TB/s HBM,
 * 5.0 PFLOP/s dense FP8), and two probes of the hardware operations the
 * MoE kernels rely on (the MFMA's accumulation inside one instruction; the
 * f32 -> bf16 and f32 -> e4m3 conversions).  Not part of the MoE forward;
 * the benchmark and the tests call them beside it.
 *
 * Conventions as in moe_fp8.h: device pointers owned by the caller, work
 * enqueued asynchronously on `stream` (NULL = default stream), arguments
 * checked on the host before any HIP call, MOE_OK or a negative MOE_ERR_*
 * code returned.  No entry point allocates.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#include "moe_fp8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Load modes of moe_peak_stream_read. */
#define MOE_PEAK_READ_PLAIN 0        /* ordinary 16-byte loads */
#define MOE_PEAK_READ_NONTEMPORAL 1  /* 16-byte loads marked nontemporal, as the
                                        GEMM kernels read weights */

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a positive
 * multiple of 16): `blocks` workgroups of 256 lanes stride over the buffer,
 * each lane keeping `unroll` (4 or 8) 16-byte loads in flight, and fold
 * every 32-bit word into an XOR.  Wave w of workgroup b writes its XOR to
 * out[4 b + w], so the XOR of out[0 .. 4 blocks) equals the XOR of all words
 * of the buffer (the check that every byte was read).
 *   out: uint32 [4 * blocks], written.  1 <= blocks <= 65536.
 * Errors: MOE_ERR_INVALID_ARG (null pointer, misaligned buf, bytes not a
 * positive multiple of 16, blocks or unroll or mode out of range),
 * MOE_ERR_NOT_GFX950, MOE_ERR_HIP. */
int moe_peak_stream_read(const void* buf, size_t bytes, int32_t blocks, int32_t unroll,
                         int32_t mode, uint32_t* out, void* stream);

/* Dense FP8 MFMA loop: `blocks` workgroups of 4 waves; each wave runs
 * `iters` rounds of 8 independent v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3,
 * f32 accumulate) on operands held in registers, the same instruction the
 * GEMM kernels use.  A operand = 1.0 in every byte, B operand = 0.5, so each
 * instruction adds 64 to every accumulator element; each lane writes the sum
 * of its 8 x 4 accumulator values, 8 * 4 * 64 * iters (exact in f32 for
 * iters <= 2048), to out[lane's global index].
 * FLOP per call = blocks * 4 * iters * 8 * (2 * 16 * 16 * 128).
 *   out: float [256 * blocks], written.  1 <= blocks <= 65536,
 *   1 <= iters <= 2048.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_NOT_GFX950, MOE_ERR_HIP. */
int moe_peak_mfma_fp8(int32_t blocks, int32_t iters, float* out, void* stream);

/* Probe modes of moe_probe_mfma_block. */
#define MOE_PROBE_E4M3 0       /* v_mfma_f32_16x16x128_f8f6f4, e4m3 x e4m3 */
#define MOE_PROBE_E4M3_E2M1 1  /* the block-scaled form, e4m3 x e2m1, UE8M0 per 32 */

/* Precision probe of the GEMMs' matrix instruction: for each of n_tiles
 * tiles, D = A B^T over one 128-wide K block with C = 0, the operands loaded
 * from memory exactly as the GEMM kernels load them.  The MoE parity tests
 * compare D with the exact dot products to measure how far the hardware's
 * accumulation inside one instruction is from the exact sum (the error the
 * oracle's exact block sums do not have).
 *   mode MOE_PROBE_E4M3:      a [n_tiles,16,128] e4m3, b [n_tiles,16,128] e4m3
 *                             (row n of b = output column n); sa, sb unused
 *   mode MOE_PROBE_E4M3_E2M1: a as above, b [n_tiles,16,64] packed e2m1
 *                             (element k in byte k/2, even k in the low
 *                             nibble), sa / sb [n_tiles,16,4] UE8M0 codes of
 *                             the four 32-wide K blocks of each row / column
 *   out float [n_tiles,16,16], out[t][m][n] = sum_k A[t][m][k] B[t][n][k]
 *                             (times the block scales), written.
 * a and b 16-byte aligned; 1 <= n_tiles <= 2^20.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_NOT_GFX950, MOE_ERR_HIP. */
int moe_probe_mfma_block(int32_t mode, int32_t n_tiles, const uint8_t* a, const uint8_t* b,
                         const uint8_t* sa, const uint8_t* sb, float* out, void* stream);

/* Exhaustive check of the two conversions the epilogues rely on, over all
 * 2^32 f32 bit patterns: the library's f32 -> bf16 (gfx950's
 * v_cvt_pk_bf16_f32) against round-to-nearest-even on the integer bits (a
 * NaN quieted with its payload kept), and the hardware f32 -> e4m3 against
 * the integer encoder of the requantisation.  `blocks` workgroups of 256
 * lanes; lane t of the N = 256 * blocks lanes takes patterns t, t + N, ...
 * and writes its mismatch counts to counts[t] (bf16) and counts[N + t]
 * (e4m3); all zero means the conversions agree everywhere.
 *   counts: uint32 [2 * 256 * blocks], written.  1 <= blocks <= 65536.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_NOT_GFX950, MOE_ERR_HIP. */
int moe_probe_conversions(int32_t blocks, uint32_t* counts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
