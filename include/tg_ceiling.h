/*
 * tg_ceiling.h — measurement entry points of libtg_gemm.so: the rate the
 * matrix cores sustain on their own, with no memory traffic, and the rate a
 * streaming read of HBM reaches.
 *
 * The GEMM of tg_gemm.h is judged against the dense fp16 matrix-core peak.
 * That peak assumes the shader clock at its maximum; with random operands
 * the power limit lowers the clock, and a kernel doing nothing but matrix
 * multiply-accumulates shows what the part delivers under that limit
 * ("TIRx 与高性能GEMM (上)" measures its kernels against the matrix unit's
 * throughput; this gives that throughput on this part, for the operand data
 * the GEMM sees).
 *
 * Not part of the GEMM path: the GEMM never calls it.
 */
#ifndef TG_CEILING_H
#define TG_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * tg_mfma_ceiling — enqueue one launch of the matrix-core stream.
 *
 *   shape       16: v_mfma_f32_16x16x32_f16, 32: v_mfma_f32_32x32x16_f16
 *               (the two shapes the GEMM kernels use).
 *   A, B        device pointers to binary16 data of a_elems and b_elems
 *               elements (each at least 8 and a multiple of 8, 16-byte
 *               aligned).  Every wave loads its operand registers once from
 *               them (wave w, register set i, lane l reads the 8 elements at
 *               ((w·16 + i)·64 + l)·8 mod a_elems, likewise for B), so the
 *               stream multiplies the caller's data: pass the GEMM's A and B
 *               for its distribution, or zeros for the unthrottled rate.
 *   waves_per_simd  1 (one workgroup of four waves per compute unit).
 *   iters       loop iterations; each wave issues 64 MFMAs of 16x16x32 (or
 *               32 of 32x32x16, two passes over 16 accumulators) per
 *               iteration on 256 fp32 accumulators held in registers:
 *               2^20 flop per wave per iteration either way.
 *   workgroups  workgroups of four waves (normally the compute-unit count).
 *   out         device pointer to workgroups·256 floats: each lane writes
 *               the sum of its accumulators (keeps the work observable).
 *   stream      hipStream_t (NULL: the null stream).
 *
 * Flop per launch: workgroups · 4 · iters · 2^20.  Returns TG_OK,
 * TG_ERR_INVALID_ARG (a bad shape, a NULL pointer, a_elems or b_elems below
 * 8 or not a multiple of 8, iters < 1, workgroups < 1, waves_per_simd != 1),
 * TG_ERR_DEVICE or TG_ERR_LAUNCH.  Asynchronous.
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

#ifdef __cplusplus
}
#endif

#endif /* TG_CEILING_H */
