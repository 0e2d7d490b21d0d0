/*
 * tg_ceiling.h — measurement entry points of libtg_gemm.so: the rate the
 * matrix cores sustain on their own, with no memory traffic, and the rate a
 * streaming read of HBM reaches.
 *
 * The GEMMs of tg_gemm.h are measured against the dense matrix-core peaks
 * (fp16 and bf16 2.5 PFLOP/s, fp8 5 PFLOP/s).  Those peaks assume the
 * shader clock at its maximum; with random operands
 * the power limit lowers the clock, and a kernel doing nothing but matrix
 * multiply-accumulates shows what the part delivers under that limit
 * ("TIRx 与高性能GEMM (上)" measures its kernels against the matrix unit's
 * throughput; this gives that throughput on this part, for the operand data
 * the GEMM sees).
 *
 * Also a stamping form of the persistent fp16 GEMM that records when each
 * workgroup starts and ends and on which XCD it runs.
 *
 * Not part of the GEMM path: the GEMM never calls these.
 */
#ifndef TG_CEILING_H
#define TG_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The instruction a matrix-core stream issues (the `shape` argument). */
#define TG_MFMA_F16_16X16X32 16   /* v_mfma_f32_16x16x32_f16: the fp16 256x256 kernels */
#define TG_MFMA_F16_32X32X16 32   /* v_mfma_f32_32x32x16_f16: the other fp16 tiles */
#define TG_MFMA_BF16_16X16X32 17  /* v_mfma_f32_16x16x32_bf16: the bf16 256x256 kernels */
#define TG_MFMA_MXF8_32X32X64 64  /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3: block-scaled FP8 */

/*
 * tg_mfma_ceiling — enqueue one launch of the matrix-core stream.
 *
 *   shape       one of the TG_MFMA_* codes above.
 *   A, B        device pointers to a_elems and b_elems elements of the
 *               instruction's input type (binary16, bfloat16 or e4m3 bytes),
 *               16-byte aligned; each count a positive multiple of 8 (16-bit
 *               types) or 32 (e4m3).  Every wave loads its operand registers
 *               once from them: fragment i of wave w, lane l is 16-byte chunk
 *               ((w·16 + i)·64 + l) of the buffer, modulo its chunk count
 *               (chunks 2c and 2c + 1 for the 32-byte e4m3 fragment c).  So
 *               the stream multiplies the caller's data: pass the GEMM's A and B
 *               for its distribution, or zeros for the unthrottled rate.  The
 *               block-scaled form runs with unit scales (E8M0 127).
 *   waves_per_simd  1 (one workgroup of four waves per compute unit).
 *   iters       loop iterations on 256 fp32 accumulators held in registers.
 *               Per wave and iteration: 64 MFMAs of 16x16x32 or 32 of
 *               32x32x16 (two passes over 16 accumulators), 2^20 flop; or 16
 *               of the block-scaled 32x32x64, 2^21 flop.
 *   workgroups  workgroups of four waves (normally the compute-unit count).
 *   out         device pointer to workgroups·256 floats: each lane writes
 *               the sum of its accumulators (keeps the work observable).
 *   stream      hipStream_t (NULL: the null stream).
 *
 * Flop per launch: workgroups · 4 · iters · 2^20 (2^21 for the block-scaled
 * form).  Returns TG_OK, TG_ERR_INVALID_ARG (an unknown shape, a NULL or
 * misaligned pointer, an element count below or not a multiple of the
 * fragment size, iters < 1, workgroups < 1, waves_per_simd != 1),
 * TG_ERR_DEVICE (not gfx950) or TG_ERR_LAUNCH.  Asynchronous.
 */
int tg_mfma_ceiling(int shape, const void *A, int64_t a_elems, const void *B, int64_t b_elems,
                    int waves_per_simd, int iters, int workgroups, float *out, void *stream);

/*
 * tg_hbm_read_ceiling — enqueue one streaming read of `bytes` bytes at src
 * (device memory, 16-byte aligned, bytes a positive multiple of 16): every
 * byte is loaded once with 16-byte non-temporal loads, four in flight per
 * lane, by `workgroups` workgroups of 256 lanes striding over the buffer.
 * The rate bytes / time is the practical HBM read bandwidth that the
 * bandwidth-bound GEMM shapes (small M: B streamed once) are held against.
 * out: device pointer to workgroups·256 unsigned words (each lane's XOR of
 * what it read, so that no load is dead).  Returns TG_OK,
 * TG_ERR_INVALID_ARG or TG_ERR_LAUNCH.  Asynchronous.
 */
int tg_hbm_read_ceiling(const void *src, int64_t bytes, int workgroups, unsigned *out, void *stream);

/*
 * tg_gemm_f16_xcd_stamps — tg_gemm_f16 for a problem that plans to the
 * persistent 256x256 kernel ("TIRx 与高性能GEMM (上)", Step 6: a fixed pool
 * of workgroups that keeps taking tiles), through an instantiation of that
 * kernel that also records, per workgroup, when it started and when all its
 * waves were done (the constant 100 MHz clock of s_memrealtime) and the XCD
 * it ran on.  D is what tg_gemm_f16 writes, bit for bit.  The spread of the
 * XCDs' last end times shows how much of a launch is one XCD finishing
 * after the others under the static tile schedule.
 *
 *   A, B, D, M, N, K, lda, ldb, ldd   as for tg_gemm_f16.
 *   stamps      device pointer to stamps_len 64-bit words; workgroup w
 *               writes words 3w (start), 3w + 1 (end), 3w + 2 (XCD id).
 *   stamps_len  at least 3 x the workgroup count (the compute-unit count
 *               rounded down to a multiple of 8, at most the tile count).
 *   workgroups  host pointer (may be NULL): the workgroup count launched.
 *   stream      hipStream_t (NULL: the null stream).
 *
 * Returns TG_OK; TG_ERR_INVALID_ARG when the arguments fail tg_gemm_f16's
 * checks, M or N is 0, the problem does not plan to the persistent kernel,
 * or stamps is NULL or too short (nothing launched); TG_ERR_TOO_LARGE,
 * TG_ERR_DEVICE or TG_ERR_LAUNCH as for tg_gemm_f16.  Asynchronous; calls
 * that overlap must not share a stamps buffer.  Measurement only: the GEMM
 * path never calls it.
 */
int tg_gemm_f16_xcd_stamps(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                           int64_t lda, int64_t ldb, int64_t ldd, uint64_t *stamps, int64_t stamps_len,
                           int64_t *workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TG_CEILING_H */
