// tg_ceiling.hip — a stream of independent matrix-core operations with no
// memory traffic, for measuring what the matrix cores sustain on their own
// under the part's power limit (declared in include/tg_ceiling.h).
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

}  // namespace

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
