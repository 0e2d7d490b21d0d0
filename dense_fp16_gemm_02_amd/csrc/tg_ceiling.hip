// tg_ceiling.hip — the two rates the GEMM kernels are held against, measured
// on the part itself (declared in include/tg_ceiling.h): a stream of
// independent matrix-core operations with no memory traffic (what the
// matrix cores sustain under the power limit), and a streaming read of HBM
// (what a read-bound kernel can reach).
//
// One workgroup of four waves per compute unit, one wave per SIMD.  Each
// wave loads its operand registers once from the caller's buffers (8 "A"
// and 8 "B" fragments of 8 16-bit values for the 16x16x32 forms, 4 + 4 for
// 32x32x16, 4 + 4 fragments of 32 e4m3 bytes for the block-scaled
// 32x32x64 form), then issues MFMAs back to back on 256 fp32 accumulators
// in registers: every MFMA of a pass writes a different accumulator, so
// none waits for another.  The operands stay in registers; successive
// MFMAs pair different fragments, so the matrix core's inputs change every
// instruction, as in the GEMM.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "tg_ceiling.h"
#include "tg_gemm.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// 16-byte chunk `idx` of a buffer of `chunks` chunks, wrapping around
__device__ inline u32x4 chunk(const u32x4 *p, int64_t chunks, int64_t idx) { return p[idx % chunks]; }

template <typename T>
__device__ inline T frag16(const u32x4 *p, int64_t chunks, int64_t idx)
{
    return __builtin_bit_cast(T, chunk(p, chunks, idx));
}

__device__ inline i32x8 frag32(const u32x4 *p, int64_t chunks, int64_t idx)
{
    const u32x4 lo = chunk(p, chunks, 2 * idx), hi = chunk(p, chunks, 2 * idx + 1);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// 16x16x32 forms (binary16 or bfloat16): 64 MFMAs of 2^14 flop per
// iteration over 8 x 8 accumulators of 4 registers.
template <typename V>
__device__ inline f4 mfma16(V a, V b, f4 c);
template <>
__device__ inline f4 mfma16<h8>(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
template <>
__device__ inline f4 mfma16<b8>(b8 a, b8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_stream_kernel(const u32x4 *__restrict__ A, int64_t a_chunks,
                                                          const u32x4 *__restrict__ B, int64_t b_chunks,
                                                          int iters, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    float s = 0.0f;
    if constexpr (KIND == TG_MFMA_F16_16X16X32 || KIND == TG_MFMA_BF16_16X16X32) {
        typedef typename std::conditional<KIND == TG_MFMA_F16_16X16X32, h8, b8>::type V;
        V fa[8], fb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            fa[i] = frag16<V>(A, a_chunks, (w * 16 + i) * 64 + lane);
            fb[i] = frag16<V>(B, b_chunks, (w * 16 + 8 + i) * 64 + lane);
        }
        f4 acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = mfma16<V>(fb[j], fa[i], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    } else {
        constexpr bool MX = KIND == TG_MFMA_MXF8_32X32X64;
        typedef typename std::conditional<MX, i32x8, h8>::type V;
        V fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (MX) {
                fa[i] = frag32(A, a_chunks, (w * 16 + i) * 64 + lane);
                fb[i] = frag32(B, b_chunks, (w * 16 + 4 + i) * 64 + lane);
            } else {
                fa[i] = frag16<h8>(A, a_chunks, (w * 16 + i) * 64 + lane);
                fb[i] = frag16<h8>(B, b_chunks, (w * 16 + 4 + i) * 64 + lane);
            }
        }
        f16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;
        // 32x32x16 binary16: two passes over the 16 accumulators, 32 MFMAs
        // of 2^15 flop (2^20 per iteration, as the 16x16x32 forms).
        // 32x32x64 e4m3 with unit block scales (E8M0 127 in every byte of
        // the scale operand): one pass, 16 MFMAs of 2^17 flop (2^21).
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int pass = 0; pass < (MX ? 1 : 2); ++pass)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (MX)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb[j], fa[i], acc[i][j], 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[(i + pass) & 3],
                                                                               acc[i][j], 0, 0, 0);
                    }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    s += acc[i][j][v];
    }
    // the lane index again from the execution mask, so that no vector
    // register carries it across the loop (all of them hold accumulators)
    const int lane_end = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    out[w * 64 + lane_end] = s;
}

// Streaming read of a buffer: 16 bytes per lane per load, four loads in
// flight per lane, grid-stride over the whole buffer; each lane folds what
// it read into one word (so no load is dead) and writes it out at the end.

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                       unsigned *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    unsigned acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int tg_hbm_read_ceiling(const void *src, int64_t bytes, int workgroups, unsigned *out, void *stream)
{
    if (!src || !out || bytes < 16 || bytes % 16 || workgroups < 1 || (uintptr_t)src % 16)
        return TG_ERR_INVALID_ARG;
    const u32x4 *p = static_cast<const u32x4 *>(src);
    int64_t n16 = bytes / 16;
    void *args[] = {(void *)&p, &n16, (void *)&out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&hbm_read_kernel), dim3((unsigned)workgroups),
                                   dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

extern "C" int tg_mfma_ceiling(int shape, const void *A, int64_t a_elems, const void *B, int64_t b_elems,
                               int waves_per_simd, int iters, int workgroups, float *out, void *stream)
{
    const void *fn = nullptr;
    int64_t esize = 2;  // bytes per element
    switch (shape) {
    case TG_MFMA_F16_16X16X32: fn = reinterpret_cast<const void *>(&mfma_stream_kernel<TG_MFMA_F16_16X16X32>); break;
    case TG_MFMA_F16_32X32X16: fn = reinterpret_cast<const void *>(&mfma_stream_kernel<TG_MFMA_F16_32X32X16>); break;
    case TG_MFMA_BF16_16X16X32:
        fn = reinterpret_cast<const void *>(&mfma_stream_kernel<TG_MFMA_BF16_16X16X32>);
        break;
    case TG_MFMA_MXF8_32X32X64:
        fn = reinterpret_cast<const void *>(&mfma_stream_kernel<TG_MFMA_MXF8_32X32X64>);
        esize = 1;
        break;
    default: return TG_ERR_INVALID_ARG;
    }
    // whole fragments: 16 bytes (8 16-bit elements) or 32 bytes (32 e4m3)
    const int64_t unit = esize == 2 ? 8 : 32;
    if (!A || !B || !out || a_elems < unit || b_elems < unit || a_elems % unit || b_elems % unit ||
        (uintptr_t)A % 16 || (uintptr_t)B % 16 || iters < 1 || workgroups < 1 || waves_per_simd != 1)
        return TG_ERR_INVALID_ARG;
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return TG_ERR_DEVICE;
    const u32x4 *a = static_cast<const u32x4 *>(A);
    const u32x4 *b = static_cast<const u32x4 *>(B);
    int64_t a_chunks = a_elems * esize / 16, b_chunks = b_elems * esize / 16;
    void *args[] = {(void *)&a, &a_chunks, (void *)&b, &b_chunks, &iters, (void *)&out};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)workgroups), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}
