// tg_gemm.hip — gfx950 kernels and the C ABI for D = A·Bᵀ (fp16 in, fp32
// accumulate, fp16 out).  See include/tg_gemm.h for the contract.
//
// Data path per workgroup (the GMEM → shared → matrix unit → register → GMEM
// path of "TIRx 基础", section "从一个最小 GEMM 开始", re-planned for CDNA4):
//   1. every thread loads 16-byte chunks of the A and B K-slices from global
//      memory into registers (coalesced along K), then writes them into an
//      XOR-swizzled LDS tile — the 128-byte swizzle of "TIRx Layout API",
//      section "示例：对 (8, 64) float16 Tile 应用 128B Swizzle";
//   2. two LDS stages form a ring across the K loop: while the matrix cores
//      consume stage s, the loads for the next K-slice are in flight and land
//      in stage s^1 ("TIRx 与高性能GEMM (上)", Step 5);
//   3. each wave reads its operand fragments with 128-bit LDS reads and issues
//      v_mfma_f32_32x32x16_f16 into fp32 accumulators held in registers;
//      the first K-slice starts from zero (the pages' accum=False);
//   4. the epilogue rounds fp32 → fp16 to nearest-even and stores only the
//      part of the tile inside M×N.
// Elements beyond M, N or K are read as zero and never written, so any shape
// works ("从编译器能力到公开算子", section "SM90a 支持具体补了什么": tail
// copies mask the valid prefix).
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tg_gemm.h"
#include "tile_layout.hpp"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;              // K elements per LDS stage (128 bytes of fp16)
constexpr int ROW_CHUNKS = BK / 8;  // 16-byte chunks per tile row

// LDS element offset of 16-byte chunk `c` (0..7) of row `r` inside a (rows × 64)
// fp16 tile.  This is ComposeLayout(per_element=3, swizzle_len=3, atom_len=3)
// over TileLayout S[(rows,64):(64@m,1@m)]; the equality is checked below at
// compile time against the layout helper.
__host__ __device__ constexpr int lds_chunk_off(int r, int c)
{
    return r * BK + ((c ^ (r & 7)) << 3);
}

static_assert(tg::layout::check_swizzled_tile(256, lds_chunk_off),
              "LDS chunk addressing disagrees with the 128B ComposeLayout swizzle");

// Fragment reads: lane l takes row (l & 31) and K-chunk (l >> 5) of a 32×16
// operand slice; the epilogue reads lane l, register v as D row (l & 31) and
// D column 8·(v/4) + 4·(l/32) + v%4 of a 32×32 tile.
__host__ __device__ constexpr int frag_row_of(int l) { return l & 31; }
__host__ __device__ constexpr int frag_hi_of(int l) { return l >> 5; }
__host__ __device__ constexpr int acc_row_of(int l, int) { return l & 31; }
__host__ __device__ constexpr int acc_col_of(int l, int v) { return 8 * (v / 4) + 4 * (l >> 5) + v % 4; }
static_assert(tg::layout::check_operand_fragment(frag_row_of, frag_hi_of),
              "operand fragment reads disagree with the MFMA operand layout");
static_assert(tg::layout::check_acc_fragment(acc_row_of, acc_col_of),
              "epilogue disagrees with the MFMA accumulator layout");

// Workgroup id → output tile.  The hardware hands workgroup w to XCD w mod 8;
// each XCD gets a contiguous range of logical tile ids, and logical ids walk
// groups of GROUP_M tile rows column by column (the grouped order of the
// pages' persistent scheduler), so the workgroups resident on one XCD share
// A and B bands in that XCD's L2.
constexpr int NUM_XCD = 8;
constexpr int GROUP_M = 8;

__host__ __device__ constexpr void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    const int xcd = bid % NUM_XCD;
    const int local = bid / NUM_XCD;
    const int per = total / NUM_XCD, rem = total % NUM_XCD;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int group_size = GROUP_M * tiles_n;
    const int group = logical / group_size;
    const int first_m = group * GROUP_M;
    const int rows_in_group = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int in_group = logical - group * group_size;
    tm = first_m + in_group % rows_in_group;
    tn = in_group / rows_in_group;
}

// Every workgroup id in [0, tiles_m·tiles_n) maps to a distinct tile inside
// the grid (checked at compile time on shapes with and without remainders).
constexpr bool tile_order_is_bijective(int tiles_m, int tiles_n)
{
    bool seen[4096] = {};
    if (tiles_m * tiles_n > 4096)
        return false;
    for (int b = 0; b < tiles_m * tiles_n; ++b) {
        int tm = -1, tn = -1;
        tile_of(b, tiles_m, tiles_n, tm, tn);
        if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n || seen[tm * tiles_n + tn])
            return false;
        seen[tm * tiles_n + tn] = true;
    }
    return true;
}
static_assert(tile_order_is_bijective(32, 56) && tile_order_is_bijective(16, 16) &&
                  tile_order_is_bijective(1, 448) && tile_order_is_bijective(4, 4) &&
                  tile_order_is_bijective(7, 9) && tile_order_is_bijective(1, 1) &&
                  tile_order_is_bijective(3, 1) && tile_order_is_bijective(13, 5) &&
                  tile_order_is_bijective(9, 17) && tile_order_is_bijective(64, 64),
              "workgroup → tile order must cover every tile exactly once");

// One 16-byte chunk (8 consecutive K) of row `row` of a K-major operand,
// zero outside rows [0,rows) or K.  VEC: 16-byte aligned rows with K % 8 == 0,
// so a chunk is either wholly inside K or wholly outside.
template <bool VEC>
__device__ inline uint4 load_chunk(const _Float16 *__restrict__ base, int64_t ld, int row,
                                   int rows, int k, int K)
{
    if constexpr (VEC) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < rows && k < K)
            v = *reinterpret_cast<const uint4 *>(base + (int64_t)row * ld + k);
        return v;
    } else {
        union {
            uint4 u;
            _Float16 h[8];
        } v;
        v.u = make_uint4(0, 0, 0, 0);
        if (row < rows) {
            const _Float16 *p = base + (int64_t)row * ld;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (k + e < K)
                    v.h[e] = p[k + e];
        }
        return v.u;
    }
}

// BM×BN workgroup tile, WM×WN waves; each wave owns a (BM/WM)×(BN/WN) block
// of D built from 32×32 MFMA tiles.  The MFMA "A" input is fed from B and
// the MFMA "B" input from A, so each lane's accumulator holds four
// consecutive columns of one row of D (see the store loop).
template <int BM, int BN, int WM, int WN, bool VEC>
__global__ __launch_bounds__(WM *WN * 64) void gemm_f16_kernel(
    const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, _Float16 *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec)
{
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int RS = NT / ROW_CHUNKS;  // rows covered by one pass of all threads
    constexpr int A_PASSES = BM / RS, B_PASSES = BN / RS;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % RS == 0 && BN % RS == 0, "tile rows must be a multiple of the load pass");
    static_assert(RS % 8 == 0, "swizzle phase must not change between load passes");
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(2 * STAGE * 2 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) _Float16 smem[2 * STAGE];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // global → LDS assignment: thread loads chunk (tid & 7) of rows
    // (tid >> 3) + p·RS, p = 0..PASSES-1
    const int lrow = tid >> 3, lch = tid & 7;
    const _Float16 *a_base = A + (int64_t)m0 * lda;
    const _Float16 *b_base = B + (int64_t)n0 * ldb;
    const int a_rows = M - m0, b_rows = N - n0;
    const int st_off = lds_chunk_off(lrow, lch);

    uint4 ra[A_PASSES], rb[B_PASSES];
    auto gload = [&](int kt) {
        const int k = kt * BK + lch * 8;
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p)
            ra[p] = load_chunk<VEC>(a_base, lda, lrow + p * RS, a_rows, k, K);
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p)
            rb[p] = load_chunk<VEC>(b_base, ldb, lrow + p * RS, b_rows, k, K);
    };
    auto lstore = [&](int s) {
        _Float16 *as = smem + s * STAGE;
        _Float16 *bs = as + BM * BK;
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p)
            *reinterpret_cast<uint4 *>(as + st_off + p * RS * BK) = ra[p];
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p)
            *reinterpret_cast<uint4 *>(bs + st_off + p * RS * BK) = rb[p];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    // fragment rows: lane reads row (lane & 31) of its 32-row tile, K-chunk
    // 2·kk + (lane >> 5) of the stage (8 consecutive K per lane)
    const int frag_row = frag_row_of(lane), frag_hi = frag_hi_of(lane);

    const int KT = (K + BK - 1) / BK;
    if (KT > 0) {
        gload(0);
        lstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < KT)
            gload(kt + 1);
        const _Float16 *as = smem + s * STAGE;
        const _Float16 *bs = as + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + frag_hi;
            f16x8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const f16x8 *>(
                    as + lds_chunk_off(wm * WTM + i * 32 + frag_row, c));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const f16x8 *>(
                    bs + lds_chunk_off(wn * WTN + j * 32 + frag_row, c));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT)
            lstore(s ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register v of lane l holds MFMA row
    // 8·(v/4) + 4·(l/32) + v%4 and MFMA column l%32; with the operand roles
    // above that is D row (l%32) and D columns 8·(v/4) + 4·(l/32) + 0..3.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = m0 + wm * WTM + i * 32 + frag_row;
        if (row >= M)
            continue;
        _Float16 *drow = D + (int64_t)row * ldd;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * WTN + j * 32 + g * 8 + frag_hi * 4;
                f16x4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (_Float16)acc[i][j][g * 4 + r];  // v_cvt_f16_f32: round to nearest even
                if (dvec && col + 3 < N) {
                    *reinterpret_cast<f16x4 *>(drow + col) = h;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (col + r < N)
                            drow[col + r] = h[r];
                }
            }
        }
    }
}

struct KernelChoice {
    const void *fn;
    const char *name;
    int bm, bn, threads;
};

template <int BM, int BN, int WM, int WN>
KernelChoice choice(bool vec, const char *name_vec, const char *name_scalar)
{
    if (vec)
        return {reinterpret_cast<const void *>(&gemm_f16_kernel<BM, BN, WM, WN, true>), name_vec,
                BM, BN, WM * WN * 64};
    return {reinterpret_cast<const void *>(&gemm_f16_kernel<BM, BN, WM, WN, false>), name_scalar,
            BM, BN, WM * WN * 64};
}

constexpr int64_t LIMIT32 = (int64_t)1 << 31;
constexpr int NUM_CU = 256;

int validate(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldd)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldd < N || lda < 0 || ldb < 0 ||
        ldd < 0)
        return TG_ERR_INVALID_ARG;
    if ((M > 0 && K > 0 && !A) || (N > 0 && K > 0 && !B) || (M > 0 && N > 0 && !D))
        return TG_ERR_INVALID_ARG;
    if (M >= LIMIT32 || N >= LIMIT32 || K >= LIMIT32 || lda >= LIMIT32 || ldb >= LIMIT32 ||
        ldd >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    return TG_OK;
}

struct Plan {
    KernelChoice k;
    int tiles_m, tiles_n;
    int dvec;
};

Plan make_plan(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldd)
{
    const bool vec = (K % 8 == 0) && (lda % 8 == 0) && (ldb % 8 == 0) &&
                     ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
    const auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    KernelChoice k;
    if (tiles(256, 256) >= NUM_CU)
        k = choice<256, 256, 2, 2>(vec, "gemm_f16_256x256_w2x2_vec", "gemm_f16_256x256_w2x2_scalar");
    else if (tiles(128, 128) >= NUM_CU)
        k = choice<128, 128, 2, 2>(vec, "gemm_f16_128x128_w2x2_vec", "gemm_f16_128x128_w2x2_scalar");
    else
        k = choice<64, 64, 2, 2>(vec, "gemm_f16_64x64_w2x2_vec", "gemm_f16_64x64_w2x2_scalar");
    Plan p;
    p.k = k;
    p.tiles_m = (int)((M + k.bm - 1) / k.bm);
    p.tiles_n = (int)((N + k.bn - 1) / k.bn);
    p.dvec = (ldd % 4 == 0) && ((uintptr_t)D % 8 == 0);
    return p;
}

// per-device "is gfx950" cache: 0 unknown, 1 yes, -1 no
std::atomic<int> g_arch_ok[64];

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return TG_ERR_DEVICE;
    if (dev < 64) {
        int s = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (s != 0)
            return s > 0 ? TG_OK : TG_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return TG_ERR_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64)
        g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? TG_OK : TG_ERR_DEVICE;
}

}  // namespace

extern "C" int tg_gemm_f16(const void *A, const void *B, void *D, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldd, void *stream)
{
    int st = validate(A, B, D, M, N, K, lda, ldb, ldd);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_OK;
    st = check_device();
    if (st != TG_OK)
        return st;
    Plan p = make_plan(A, B, D, M, N, K, lda, ldb, ldd);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
    if (grid >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    int Mi = (int)M, Ni = (int)N, Ki = (int)K;
    void *args[] = {(void *)&A, (void *)&B, (void *)&D, &Mi, &Ni, &Ki, &lda, &ldb, &ldd,
                    &p.tiles_m, &p.tiles_n, &p.dvec};
    hipError_t e = hipLaunchKernel(p.k.fn, dim3((unsigned)grid), dim3(p.k.threads), args, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

extern "C" int tg_gemm_f16_plan(const void *A, const void *B, const void *D, int64_t M,
                                int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                                char *name, int64_t name_len, int64_t *grid)
{
    int st = validate(A, B, D, M, N, K, lda, ldb, ldd);
    if (name && name_len > 0)
        name[0] = 0;
    if (grid)
        *grid = 0;
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    Plan p = make_plan(A, B, D, M, N, K, lda, ldb, ldd);
    if (name && name_len > 0)
        snprintf(name, (size_t)name_len, "%s", p.k.name);
    if (grid)
        *grid = (int64_t)p.tiles_m * p.tiles_n;
    return TG_OK;
}

extern "C" const char *tg_status_string(int status)
{
    switch (status) {
    case TG_OK:
        return "ok";
    case TG_ERR_INVALID_ARG:
        return "invalid argument (negative size, leading dimension too small, or NULL matrix)";
    case TG_ERR_LAUNCH:
        return "kernel launch failed";
    case TG_ERR_DEVICE:
        return "no usable gfx950 device";
    case TG_ERR_TOO_LARGE:
        return "dimension exceeds the 32-bit range the kernels address";
    default:
        return "unknown status";
    }
}
