/*
 * tg_gemm.h — C ABI of the MI355X (gfx950) fp16 GEMM library libtg_gemm.so.
 *
 * The operation ("TIRx 与高性能GEMM (上)", section "从 GEMM 公式到数据路径";
 * "TIRx 基础", the 128×128×64 reference kernel):
 *
 *     D = A · Bᵀ,   A: M×K,  B: N×K (weights stored row by row, so the
 *                   transpose moves no data),  D: M×N.
 *
 * Operands and result are IEEE binary16; products are accumulated in fp32
 * (the reference kernel's accumulator type) and each element of D is rounded
 * once from fp32 to binary16 with round-to-nearest-even (the cvt.rn
 * conversion of "TIRx Compiler Foundation", section "Example: A GEMM
 * Kernel").  The order of the fp32 additions is unspecified.
 *
 * All matrices are row-major with leading dimensions in elements:
 *     A[i,k] = A[i*lda + k],  B[j,k] = B[j*ldb + k],  D[i,j] = D[i*ldd + j].
 *
 * Status codes are returned by every entry point; nothing is thrown.
 */
#ifndef TG_GEMM_H
#define TG_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TG_OK = 0,
    /* negative dimension, lda < K, ldb < K, ldd < N, or a NULL pointer for a
     * matrix that has elements.  Nothing is launched. */
    TG_ERR_INVALID_ARG = -1,
    /* the HIP runtime rejected the launch (hipGetLastError after it). */
    TG_ERR_LAUNCH = -2,
    /* the current device is not a gfx950 GPU, or no device is usable. */
    TG_ERR_DEVICE = -3,
    /* a dimension or index exceeds what the kernels address (each of M, N,
     * K, lda, ldb, ldd must be below 2^31, and A, B, D must each span fewer
     * than 2^62 elements).  Nothing is launched. */
    TG_ERR_TOO_LARGE = -4,
    /* block-scaled entry points only: K is not a multiple of 32, lda or
     * ldb not a multiple of 16, ldsa or ldsb not a multiple of 4, A or B
     * not 16-byte aligned, or SA or SB not 4-byte aligned (16-byte for the
     * packed layout; tg_mx_pack_scales: P not 16-byte aligned).  Nothing is
     * launched. */
    TG_ERR_LAYOUT = -5
};

/*
 * tg_gemm_f16 — D ← fp16_rne(A · Bᵀ) over the M×N window of D.
 *
 *   A, B, D   device pointers (hipMalloc'd or equivalent) to binary16 data.
 *             A is read over rows [0,M) and columns [0,K); B over rows [0,N)
 *             and columns [0,K); D is written over rows [0,M) and columns
 *             [0,N) only — elements of D outside that window, and padding
 *             columns of A and B beyond K, are never touched.  D must not
 *             overlap A or B (not checked).
 *   M, N, K   problem size.  M == 0 or N == 0: returns TG_OK, nothing
 *             launched.  K == 0: D's window is set to +0.
 *   lda, ldb  leading dimensions of A and B in elements, >= K.
 *   ldd       leading dimension of D in elements, >= N.
 *   stream    a hipStream_t (NULL = the null stream).  The call only
 *             enqueues work and returns; the caller synchronizes.
 *
 * There is no alpha/beta: D's prior contents are ignored.  Any alignment is
 * accepted; 16-byte-aligned A/B with K, lda, ldb multiples of 8 take the
 * vector-load path, other inputs a slower element-wise path with the same
 * results.  The library allocates nothing, keeps no state between calls
 * (beyond a per-device cache of the device's attributes) and is safe to
 * call from several host threads.  A call only launches kernels — no
 * allocation, memset or synchronization — so it may be recorded into a HIP
 * graph under stream capture and replayed.  Kernel faults surface at the
 * caller's next synchronization.  From 4 MiB of D on (16-byte aligned rows),
 * most of D is written with non-temporal stores: it is not kept in the
 * caches for a consumer that reads it right after the call.
 *
 * Returns TG_OK, TG_ERR_INVALID_ARG, TG_ERR_TOO_LARGE, TG_ERR_DEVICE or
 * TG_ERR_LAUNCH.
 */
int tg_gemm_f16(const void *A, const void *B, void *D,
                int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldd,
                void *stream);

/*
 * tg_gemm_f16_plan — host-only: the name of the kernel tg_gemm_f16 would
 * launch for these arguments, and the number of output tiles it splits D
 * into, without touching the device.  Writes a NUL-terminated name of at
 * most `name_len` bytes into `name` (may be NULL) and the tile count into
 * *tiles (may be NULL; 0 when nothing would be launched); the launch has
 * one workgroup per tile.  Returns the status tg_gemm_f16 would return for
 * argument validation (TG_OK, TG_ERR_INVALID_ARG or TG_ERR_TOO_LARGE).
 */
int tg_gemm_f16_plan(const void *A, const void *B, const void *D,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldd,
                     char *name, int64_t name_len, int64_t *tiles);

/*
 * tg_gemm_bf16 — the same operation on bfloat16 data: D = A·Bᵀ with A, B and
 * D bfloat16 (bit patterns in 2-byte elements, same layout, strides, edge
 * cases, streams, threading and return codes as tg_gemm_f16), products
 * accumulated in fp32 and the result rounded to bfloat16 to nearest even.
 * "从编译器能力到公开算子", section "SM90a 支持具体补了什么": the matrix
 * path takes FP16 or BF16 inputs with FP32 accumulation; the pages name no
 * BF16 output rounding, and round-to-nearest-even (the fp16 epilogue's
 * cvt.rn) is the reading taken.
 */
int tg_gemm_bf16(const void *A, const void *B, void *D,
                 int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldd,
                 void *stream);

/* tg_gemm_bf16_plan — tg_gemm_f16_plan for tg_gemm_bf16 (names start with
 * "gemm_bf16_"). */
int tg_gemm_bf16_plan(const void *A, const void *B, const void *D,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldd,
                      char *name, int64_t name_len, int64_t *tiles);

/*
 * tg_gemm_mxf8 — block-scaled FP8 GEMM:
 *
 *   D[i,j] ← fp16_rne( Σ_k (2^(SA[i,k/32]-127)·A[i,k]) · (2^(SB[j,k/32]-127)·B[j,k]) )
 *
 * "TIRx Layout API", section "Scale Factor 布局": a block-scaled MMA reads
 * one 8-bit scale factor per group of K elements of every row besides its
 * operands (the page's example is a block-scaled FP8 GEMM).  The pages fix
 * neither the encodings nor the group length; this entry point takes the
 * OCP MX reading: A and B hold FP8 E4M3 codes (bias 7, no infinities,
 * S.1111.111 is NaN, largest finite 448), and every 32 consecutive K elements
 * of a row share one UE8M0 scale byte worth 2^(s-127) (255 is NaN).  Products
 * are accumulated in fp32 and D is binary16, rounded to nearest even.
 *
 *   A    device pointer, M×K bytes, row i at A + i·lda; 16-byte aligned.
 *   SA   device pointer, M×ldsa scale bytes, SA[i,b] = SA[i·ldsa + b] for
 *        blocks b < K/32; 4-byte aligned.  Bytes past K/32 in a row are
 *        never used (they may hold anything).
 *   B    device pointer, N×K bytes (the weight, stored like A), row j at
 *        B + j·ldb; 16-byte aligned.
 *   SB   device pointer, N×ldsb scale bytes, like SA.
 *   D    device pointer to binary16, M×N window with leading dimension ldd
 *        (elements); written only inside the window.
 *   K    a multiple of 32 (whole scale blocks); K == 0 sets D's window to +0.
 *   lda, ldb   bytes between rows, >= K and multiples of 16.
 *   ldsa, ldsb bytes between scale rows, >= K/32 and multiples of 4.
 *   stream     as for tg_gemm_f16.
 *
 * Ownership, threading, asynchrony, edge cases in M and N and the
 * non-temporal writing of a large D are as for tg_gemm_f16.  Returns TG_OK,
 * TG_ERR_INVALID_ARG (negative sizes, a
 * leading dimension too small, a NULL pointer with elements behind it),
 * TG_ERR_LAYOUT (the multiple-of and alignment rules above),
 * TG_ERR_TOO_LARGE, TG_ERR_DEVICE or TG_ERR_LAUNCH.
 */
int tg_gemm_mxf8(const void *A, const void *SA, const void *B, const void *SB, void *D,
                 int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd,
                 void *stream);

/* tg_gemm_mxf8_plan — host-only: the kernel name ("gemm_mxf8_…") and tile
 * count tg_gemm_mxf8 would use, and its argument-validation status; outputs
 * as for tg_gemm_f16_plan. */
int tg_gemm_mxf8_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd,
                      char *name, int64_t name_len, int64_t *tiles);

/*
 * Packed scale layout.  The page's scale-factor layout ("TIRx Layout API",
 * section "Scale Factor 布局") is built from an atom of 32 rows × the scale
 * factors one MMA reads, repeated along M and along the K scale blocks.
 * The packed layout stores scales the same way in device memory: 512-byte
 * chunks of 32 rows × 16 blocks (512 elements of K), so that the scale
 * bytes a 32-row operand fragment needs for four 128-K tiles are 512
 * contiguous bytes rather than one cache line per row.  For R rows and K
 * (a multiple of 32), with G = ceil(K/512) chunks per 32-row group:
 *
 *   byte of row r, block b  at  ((r/32)·G + b/16)·512 + (r%32)·16 + b%16
 *
 * and the buffer holds ceil(R/32)·G·512 bytes (tg_mx_packed_bytes).  Bytes
 * for rows >= R or blocks >= K/32 are never used (tg_mx_pack_scales writes
 * 127 there).
 *
 * tg_mx_packed_bytes — the size of that buffer for `rows` rows and K; -1 if
 * rows or K is negative, K is not a multiple of 32, or either is >= 2^31.
 */
int64_t tg_mx_packed_bytes(int64_t rows, int64_t K);

/*
 * tg_mx_pack_scales — enqueue the conversion of row-major scales (rows ×
 * K/32 bytes, row r at S + r·lds, as tg_gemm_mxf8 takes them) into the
 * packed layout at P (device memory of tg_mx_packed_bytes(rows, K) bytes,
 * 16-byte aligned, not overlapping S).  A layout change only: every byte
 * is copied unchanged.  Returns TG_OK (nothing to do for rows == 0 or
 * K == 0), TG_ERR_INVALID_ARG (negative sizes, K not a multiple of 32,
 * lds < K/32, a NULL pointer with bytes behind it), TG_ERR_LAYOUT (P not
 * 16-byte aligned), TG_ERR_TOO_LARGE (rows, K or lds >= 2^31),
 * TG_ERR_DEVICE or TG_ERR_LAUNCH.  Asynchronous on `stream`.
 */
int tg_mx_pack_scales(const void *S, int64_t rows, int64_t K, int64_t lds, void *P, void *stream);

/*
 * tg_gemm_mxf8_packed — tg_gemm_mxf8 with both scale matrices in the packed
 * layout (SA for M rows, SB for N rows, each 16-byte aligned; no scale
 * leading dimensions).  Same arithmetic, the same kernels (they differ only
 * in where a scale word is read), so D is bit-identical to tg_gemm_mxf8 on
 * the same scales.  A caller whose scales are fixed (a weight's) packs them
 * once; the block-scaled kernels then read each fragment's scale words for
 * four K-tiles from 512 contiguous bytes.  Arguments, ownership and status
 * codes as for tg_gemm_mxf8; TG_ERR_LAYOUT also when SA or SB is not
 * 16-byte aligned; TG_ERR_TOO_LARGE also for K >= 2^27 (the packed
 * offsets inside one workgroup's rows stay below 2^31).
 */
int tg_gemm_mxf8_packed(const void *A, const void *SA, const void *B, const void *SB, void *D,
                        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                        void *stream);

/* tg_gemm_mxf8_packed_plan — host-only: the kernel name ("gemm_mxf8p_…")
 * and tile count tg_gemm_mxf8_packed would use, and its validation status;
 * outputs as for tg_gemm_f16_plan. */
int tg_gemm_mxf8_packed_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                             char *name, int64_t name_len, int64_t *tiles);

/*
 * Element encodings of the block-scaled GEMM.  The pages name the
 * block-scaled FP8 GEMM ("TIRx Layout API", section "Scale Factor 布局")
 * without fixing its element encoding; OCP MX defines two FP8 element
 * encodings; tg_gemm_mxf8 and tg_gemm_mxf8_packed take E4M3 on both
 * operands, tg_gemm_mx and tg_gemm_mx_packed take either on each:
 *   TG_MX_E4M3  sign, 4 exponent bits (bias 7), 3 fraction bits; no
 *               infinities, S.1111.111 is NaN, largest finite 448.
 *   TG_MX_E5M2  sign, 5 exponent bits (bias 15), 2 fraction bits; exponent
 *               31 is ±infinity (fraction 0) or NaN, largest finite 57344
 *               (the upper byte of a binary16 pattern).
 * Infinite or NaN elements and scales propagate through the fp32 sum as IEEE
 * arithmetic has them (infinity times zero is NaN); a result past binary16's
 * range is ±infinity.
 */
enum { TG_MX_E4M3 = 0, TG_MX_E5M2 = 1 };

/*
 * tg_gemm_mx — tg_gemm_mxf8 with the element encoding of A (a_format) and of
 * B (b_format) chosen separately among TG_MX_E4M3 and TG_MX_E5M2 (the same
 * scale bytes, layouts, kernels and status codes; any other format value is
 * TG_ERR_INVALID_ARG).  tg_gemm_mx with both formats TG_MX_E4M3 is
 * tg_gemm_mxf8.  tg_gemm_mx_plan, tg_gemm_mx_packed and
 * tg_gemm_mx_packed_plan extend tg_gemm_mxf8_plan, tg_gemm_mxf8_packed and
 * tg_gemm_mxf8_packed_plan the same way; a plan's kernel name carries the
 * encodings as a suffix ("_e5m2" for both E5M2, "_e5m2xe4m3" for A E5M2 and
 * B E4M3, "_e4m3xe5m2" for the reverse; none for E4M3 on both).
 */
int tg_gemm_mx(const void *A, const void *SA, const void *B, const void *SB, void *D,
               int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd,
               int a_format, int b_format, void *stream);
int tg_gemm_mx_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                    int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd,
                    int a_format, int b_format, char *name, int64_t name_len, int64_t *tiles);
int tg_gemm_mx_packed(const void *A, const void *SA, const void *B, const void *SB, void *D,
                      int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                      int a_format, int b_format, void *stream);
int tg_gemm_mx_packed_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                           int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                           int a_format, int b_format, char *name, int64_t name_len, int64_t *tiles);

/* tg_status_string — a static, NUL-terminated description of a status. */
const char *tg_status_string(int status);

/* tg_device_info — the current device's compute-unit count, its maximum
 * shader clock in kHz and its architecture name (NUL-terminated, truncated
 * to arch_len bytes; arch may be NULL).  Lets a caller derive the dense
 * matrix-core peak as CUs × flop per clock per CU × clock, the figure the
 * peak percentages of the measurements rest on.  Outputs are written only on
 * success; NULL output pointers are skipped.  Host-only, synchronous, no
 * kernel launch.  Returns TG_OK, or TG_ERR_DEVICE if no device is
 * available or a runtime query fails. */
int tg_device_info(int *compute_units, int *max_clock_khz, char *arch, int64_t arch_len);

#ifdef __cplusplus
}
#endif

#endif /* TG_GEMM_H */
