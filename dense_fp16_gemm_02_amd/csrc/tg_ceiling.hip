// tg_ceiling.hip — the two rates the GEMM kernels are held against, measured
// on the part itself (declared in include/tg_ceiling.h): a stream of
// independent matrix-core operations with no memory traffic (what the
// matrix cores sustain under the power limit), and a streaming read of HBM
// (what a read-bound kernel can reach).
//
// One workgroup of four waves per compute unit, one wave per SIMD.  Each
// wave loads 16 operand registers of 8 binary16 values (8 "A" and 8 "B"
// fragments for the 16x16x32 form, 4 + 4 for 32x32x16) once from the
// caller's buffers, then issues MFMAs back to back on 256 fp32 accumulators
// in registers: every MFMA of an iteration writes a different accumulator,
// so none waits for another.  The operands stay in registers; successive
// MFMAs pair different fragments, so the matrix core's inputs change every
// instruction, as in the GEMM.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "tg_ceiling.h"
#include "tg_gemm.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ inline h8 load_frag(const _Float16 *p, int64_t elems, int64_t idx)
{
    return *reinterpret_cast<const h8 *>(p + (idx * 8) % elems);
}

template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_stream_kernel(const _Float16 *__restrict__ A, int64_t a_elems,
                                                          const _Float16 *__restrict__ B, int64_t b_elems,
                                                          int iters, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    constexpr int NF = SHAPE == 16 ? 8 : 4;  // fragments per operand
    h8 fa[NF], fb[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        fa[i] = load_frag(A, a_elems, (w * 16 + i) * 64 + lane);
        fb[i] = load_frag(B, b_elems, (w * 16 + NF + i) * 64 + lane);
    }
    float s = 0.0f;
    if constexpr (SHAPE == 16) {
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
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    } else {
        f16v acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;
        // two passes over the 16 accumulators: 32 MFMAs of 2^15 flop, the
        // same 2^20 flop per iteration as the 16x16x32 form
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int pass = 0; pass < 2; ++pass)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[(i + pass) & 3], acc[i][j],
                                                                           0, 0, 0);
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
    if ((shape != 16 && shape != 32) || !A || !B || !out || a_elems < 8 || b_elems < 8 || a_elems % 8 ||
        b_elems % 8 || iters < 1 || workgroups < 1 || waves_per_simd != 1)
        return TG_ERR_INVALID_ARG;
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return TG_ERR_DEVICE;
    const void *fn = shape == 16 ? reinterpret_cast<const void *>(&mfma_stream_kernel<16>)
                                 : reinterpret_cast<const void *>(&mfma_stream_kernel<32>);
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    void *args[] = {(void *)&a, &a_elems, (void *)&b, &b_elems, &iters, (void *)&out};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)workgroups), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}
