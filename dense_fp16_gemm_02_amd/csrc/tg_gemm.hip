// tg_gemm.hip — gfx950 kernels and the C ABI for D = A·Bᵀ (fp16 in, fp32
// accumulate, fp16 out).  See include/tg_gemm.h for the contract.
//
// Data path per workgroup (the GMEM → shared → matrix unit → register → GMEM
// path of "TIRx 基础", section "从一个最小 GEMM 开始", re-planned for CDNA4):
//   1. the A and B K-slices move from global memory straight into LDS by
//      direct-to-LDS buffer loads (16 bytes per lane, coalesced along K); the
//      XOR swizzle of "TIRx Layout API", section "示例：对 (8, 64) float16
//      Tile 应用 128B Swizzle", re-derived for a 64-bank LDS, is applied on
//      the source side (operands that are not 16-byte aligned go through
//      registers instead);
//   2. LDS stages form rings across the K loop: while the matrix cores
//      consume one stage, the loads of the next K-slices are in flight into
//      the others ("TIRx 与高性能GEMM (上)", Step 5; the largest tile keeps
//      three stages of A and two of B);
//   3. each wave reads its operand fragments with 128-bit LDS reads and issues
//      v_mfma_f32_16x16x32_f16 (largest tile) or v_mfma_f32_32x32x16_f16 into
//      fp32 accumulators held in registers; the first K-slice starts from
//      zero (the pages' accum=False);
//   4. the epilogue rounds fp32 → fp16 to nearest-even, stages the tile in
//      LDS and stores the part inside M×N in 16-byte row segments.
// Elements beyond M, N or K are read as zero and never written, so any shape
// works ("从编译器能力到公开算子", section "SM90a 支持具体补了什么": tail
// copies mask the valid prefix).
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tg_gemm.h"
#include "tile_layout.hpp"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element type of A, B and D: binary16 or bfloat16.  Both take the same
// tiles, DMAs and LDS layouts (2-byte elements); they differ only in the
// MFMA that consumes the fragments and in the fp32 → element conversion of
// the epilogue (a C cast: round to nearest even for both).
template <typename E>
struct Elem;
template <>
struct Elem<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
    static constexpr const char *prefix = "gemm_f16_";
    __device__ static f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elem<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
    static constexpr const char *prefix = "gemm_bf16_";
    __device__ static f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }

constexpr int BK = 64;              // K elements per LDS stage (128 bytes of fp16)
constexpr int ROW_CHUNKS = BK / 8;  // 16-byte chunks per tile row

// LDS element offset of 16-byte chunk `c` (0..7) of row `r` inside a (rows × 64)
// fp16 tile: ComposeLayout(per_element=3, swizzle_len=3, atom_len=4) over
// TileLayout S[(rows,64):(64@m,1@m)] — the pages' 128-byte swizzle keeps
// 16-byte vectors whole and XORs the row into the chunk index; here the XOR
// takes the row pair (r >> 1) instead of the row, because gfx950's LDS has 64
// four-byte banks and serves a 128-bit read 16 lanes at a time: sixteen
// consecutive rows (one MFMA fragment read's first 16 lanes) must then hit
// sixteen different 16-byte bank groups, which the 128-byte mode misses by a
// factor of two (rows r and r+8 collide).  Checked at compile time against
// the layout helper.
constexpr int SWZ_ROW_SHIFT = 1;
__host__ __device__ constexpr int swz(int r) { return (r >> SWZ_ROW_SHIFT) & 7; }
__host__ __device__ constexpr int lds_chunk_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

static_assert(tg::layout::check_swizzled_tile(tg::layout::swizzle_pairs_f16(256), 256, 64, lds_chunk_off),
              "LDS chunk addressing disagrees with ComposeLayout(3, 3, 4)");

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

// The same for v_mfma_f32_16x16x32_f16: lane l takes row (l & 15) and
// K-chunk (l >> 4) of a 16×32 operand slice; register v of lane l is D row
// (l & 15), D column 4·(l >> 4) + v of a 16×16 tile.
__host__ __device__ constexpr int frag16_row_of(int l) { return l & 15; }
__host__ __device__ constexpr int frag16_hi_of(int l) { return l >> 4; }
__host__ __device__ constexpr int acc16_row_of(int l, int) { return l & 15; }
__host__ __device__ constexpr int acc16_col_of(int l, int v) { return 4 * (l >> 4) + v; }
static_assert(tg::layout::check_operand_fragment(frag16_row_of, frag16_hi_of,
                                                 tg::layout::mfma16x16x32_operand(), 32),
              "operand fragment reads disagree with the 16x16x32 MFMA operand layout");
static_assert(tg::layout::check_acc_fragment(acc16_row_of, acc16_col_of, tg::layout::mfma16x16_acc_swapped(), 16),
              "epilogue map disagrees with the 16x16 MFMA accumulator layout");

// Workgroup id → output tile.  The hardware hands workgroup w to XCD w mod 8;
// each XCD gets a contiguous range of logical tile ids, and logical ids walk
// groups of GROUP_M tile rows column by column (the grouped order of the
// pages' persistent scheduler), so the workgroups resident on one XCD share
// A and B bands in that XCD's L2; group g starts its column walk at column
// g·tiles_n/8.
constexpr int NUM_XCD = 8;
#ifndef TG_GROUP_M
#define TG_GROUP_M 4
#endif
constexpr int GROUP_M = TG_GROUP_M;

template <int GM>
__host__ __device__ constexpr void tile_of_grouped(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int GROUP_M = GM;
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
    // Each group walks the columns from its own starting point, spread over
    // the row of tiles, so that the XCDs (which hold consecutive groups)
    // stream different B bands at any moment rather than all requesting the
    // same one.
    const int start = (int)((int64_t)group * tiles_n / NUM_XCD % tiles_n);
    tn = in_group / rows_in_group + start;
    if (tn >= tiles_n)
        tn -= tiles_n;
}

__host__ __device__ constexpr void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    tile_of_grouped<GROUP_M>(bid, tiles_m, tiles_n, tm, tn);
}

// Every workgroup id in [0, tiles_m·tiles_n) maps to a distinct tile inside
// the grid (checked at compile time on shapes with and without remainders).
template <int GM = GROUP_M>
constexpr bool tile_order_is_bijective(int tiles_m, int tiles_n)
{
    bool seen[4096] = {};
    if (tiles_m * tiles_n > 4096)
        return false;
    for (int b = 0; b < tiles_m * tiles_n; ++b) {
        int tm = -1, tn = -1;
        tile_of_grouped<GM>(b, tiles_m, tiles_n, tm, tn);
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
static_assert(tile_order_is_bijective<8>(32, 56) && tile_order_is_bijective<8>(16, 16) &&
                  tile_order_is_bijective<8>(1, 448) && tile_order_is_bijective<8>(7, 9) &&
                  tile_order_is_bijective<8>(17, 33) && tile_order_is_bijective<8>(9, 17) &&
                  tile_order_is_bijective<8>(64, 64) && tile_order_is_bijective<8>(3, 1),
              "workgroup → tile order (groups of 8 tile rows) must cover every tile exactly once");

// One 16-byte chunk (8 consecutive K) of row `row` of a K-major operand,
// zero outside rows [0,rows) or K.  VEC: 16-byte aligned rows with K % 8 == 0,
// so a chunk is either wholly inside K or wholly outside.
template <bool VEC, typename E>
__device__ inline uint4 load_chunk(const E *__restrict__ base, int64_t ld, int row,
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
            E h[8];
        } v;
        v.u = make_uint4(0, 0, 0, 0);
        if (row < rows) {
            const E *p = base + (int64_t)row * ld;
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
template <typename E, int BM, int BN, int WM, int WN, bool VEC>
__global__ __launch_bounds__(WM *WN * 64) void gemm_vec_kernel(
    const E *__restrict__ A, const E *__restrict__ B, E *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec)
{
    using V8 = typename Elem<E>::v8;
    using V4 = typename Elem<E>::v4;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int RS = NT / ROW_CHUNKS;  // rows covered by one pass of all threads
    constexpr int A_PASSES = BM / RS, B_PASSES = BN / RS;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % RS == 0 && BN % RS == 0, "tile rows must be a multiple of the load pass");
    static_assert(RS % 16 == 0, "swizzle phase must not change between load passes");
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(2 * STAGE * 2 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) E smem[2 * STAGE];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // global → LDS assignment: thread loads chunk (tid & 7) of rows
    // (tid >> 3) + p·RS, p = 0..PASSES-1
    const int lrow = tid >> 3, lch = tid & 7;
    const E *a_base = A + (int64_t)m0 * lda;
    const E *b_base = B + (int64_t)n0 * ldb;
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
        E *as = smem + s * STAGE;
        E *bs = as + BM * BK;
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
        const E *as = smem + s * STAGE;
        const E *bs = as + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + frag_hi;
            V8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const V8 *>(
                    as + lds_chunk_off(wm * WTM + i * 32 + frag_row, c));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const V8 *>(
                    bs + lds_chunk_off(wn * WTN + j * 32 + frag_row, c));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = Elem<E>::mfma(bf[j], af[i], acc[i][j]);
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
        E *drow = D + (int64_t)row * ldd;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * WTN + j * 32 + g * 8 + frag_hi * 4;
                V4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (E)acc[i][j][g * 4 + r];  // v_cvt_f16_f32: round to nearest even
                if (dvec && col + 3 < N) {
                    *reinterpret_cast<V4 *>(drow + col) = h;
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

typedef __attribute__((address_space(3))) void *lds_void_ptr;

// Intended waves per SIMD of a kernel (OCC workgroups of four waves per
// CU): lets the register allocator spend up to 512/OCC registers per wave
// (device compile only; the host pass does not know the attribute).
#if defined(__HIP_DEVICE_COMPILE__)
#define TG_WAVES_PER_SIMD(n) __attribute__((amdgpu_waves_per_eu(n, n)))
#else
#define TG_WAVES_PER_SIMD(n)
#endif

// Cache-policy bits of a DMA (the instruction's sc0/sc1/nt fields).  An
// operand that every resident workgroup re-reads stays in the default
// (cached) policy; in the column-strip tiles B is read exactly once, so its
// loads are marked non-temporal and system-coherent-level-0 (sc0 | nt): they
// stream past the caches instead of evicting A, which every strip re-reads.
// Fence after each slot's MFMA: the MFMA issues first and its companions
// (fragment reads, DMAs) issue in its shadow, never ahead of it.
#define MFMA_FIRST() __builtin_amdgcn_sched_barrier(0)
constexpr int CPOL_CACHED = 0;
constexpr int CPOL_STREAM = 1 | 2;  // sc0 | nt

// Raw buffer descriptor word 3 for gfx9-family GPUs (32-bit data format, no
// swizzle, no thread-id add).  Offsets at or past DMA_RANGE bytes read zeros.
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;
constexpr int DMA_RANGE = 0x7fffffff;
constexpr uint32_t DMA_OOB = 0x80000000u;

// One 16-byte-per-lane DMA: buffer bytes [voff, voff+16) of lane l land at
// LDS bytes lds + 16·l (lds must be wave-uniform).  The builtin exists only
// in the device pass; the host pass sees an empty body, which keeps clang
// emitting the host-side kernel stubs.
template <int CPOL = 0>
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, void *lds, uint32_t voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)lds, 16, voff, 0, 0, CPOL);
#else
    (void)rsrc, (void)lds, (void)voff;
#endif
}

// The direct-to-LDS path addresses a tile with 32-bit byte offsets from its
// origin (+k, which goes into the descriptor base): the largest offset it
// forms, (rows-1)·ld·2 + 16·7, must stay below DMA_RANGE.
__host__ __device__ constexpr bool dma_offsets_fit(int64_t rows, int64_t ld)
{
    return (rows - 1) * ld * 2 + 128 < (int64_t)DMA_RANGE;
}

// Wait until at most N of this wave's vector-memory operations (here: LDS
// DMAs) are outstanding.  Inline assembly, so the compiler neither drops nor
// relaxes it.
template <int N>
__device__ inline void wait_vmem()
{
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// This lane's index in its wave, computed from the execution mask rather
// than from the work-item id.  The epilogues call it after the K loop, so
// that no register has to carry a lane-derived value across the loop (with
// every VGPR of the loop taken, such values were spilled to scratch).
__device__ inline int lane_id()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Workgroup barrier that waits only for this wave's LDS reads (lgkmcnt), not
// for its in-flight DMAs as __syncthreads would; the memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ inline void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Operand tile in LDS: rows of BK_ fp16 (BK_/8 chunks of 16 bytes).  Chunk c
// of row r sits at chunk c ^ swz(r), swz(r) = (r / ROWS_PER_LINE) mod RC, with
// ROWS_PER_LINE the rows sharing one 256-byte bank line.  That is
// ComposeLayout(per_element=3, swizzle_len=log2(RC), atom_len=4) over
// S[(rows,BK_):(BK_@m,1@m)]: like the pages' 128-byte mode it keeps 16-byte
// vectors whole and XORs row bits into the chunk index, but it takes the row
// bits above the bank line, because gfx950's LDS has 64 four-byte banks and
// serves a 128-bit read 16 lanes at a time — sixteen consecutive rows (the
// first 16 lanes of an MFMA fragment read) then land on sixteen different
// 16-byte bank slots.  (The 128-byte mode, for BK_ = 64, puts rows r and r+8
// on the same banks: a measured 2-way conflict on every fragment read.)
template <int BK_>
struct OperandTile {
    static constexpr int RC = BK_ / 8;
    static constexpr int ROWS_PER_LINE = 128 / BK_;
    static constexpr int ROWS_PER_DMA = 64 / RC;  // rows one wave DMA instruction fills
    __host__ __device__ static constexpr int swz(int r) { return (r / ROWS_PER_LINE) & (RC - 1); }
    __host__ __device__ static constexpr int off(int r, int c) { return r * BK_ + ((c ^ swz(r)) << 3); }
};
static_assert(tg::layout::check_swizzled_tile(tg::layout::swizzle_bank256_f16(256, 64), 256, 64,
                                              OperandTile<64>::off),
              "BK=64 LDS addressing disagrees with ComposeLayout(3, 3, 4)");
static_assert(tg::layout::check_swizzled_tile(tg::layout::swizzle_bank256_f16(256, 32), 256, 32,
                                              OperandTile<32>::off),
              "BK=32 LDS addressing disagrees with ComposeLayout(3, 2, 4)");

// Second half of the staged epilogue: one wave's WTM×WTN block of D, held
// in LDS as row-major fp16 with the 16-byte chunk index of row r XORed with
// r mod (WTN/8) (stage_off), goes to global memory 16 bytes per lane along
// rows: lane l takes chunk l mod (WTN/8) of row l / (WTN/8), 512/WTN rows per
// pass, so each store instruction writes 64·16 bytes as whole row segments.
// A block wholly inside D with 16-byte aligned rows (dvec) issues its LDS
// reads in batches ahead of the stores, with no per-row branches; a block
// on an edge checks every row against M and every column against N.  NR
// and r0 select rows r0 .. r0+NR-1 of the block, so that an epilogue can
// stage and store its block a band of rows at a time: the first stores
// then go out while the later bands are still being converted and staged
// (in quarters: 0.8–6% faster for the one-tile 256×256 kernels; per
// fragment row: 2.5% for the producer/consumer 128×128 kernel and the
// block-scaled strips, while the small blocks of the other DMA kernels
// measured 1–2% slower that way and store theirs whole).
//
// dvec, the D store mode of the kernels with a staged epilogue: D_ELEM
// element stores, D_VEC 16-byte stores, D_VEC_NT 16-byte stores marked
// non-temporal for the blocks wholly inside D.  The host picks D_VEC_NT
// when D is large (D_NT_MIN_BYTES): written once and never read back, D then
// streams out past the caches' reuse, which measured 0.4–5% faster from 4
// MiB of D on and 5% slower on a 2 MB D (1000³), where the stores' longer
// completion is not hidden behind other work.  The non-temporal stores are
// buffer stores from the block's origin (32-bit offsets: the host checks
// that a 256-row block fits), which also keeps the compiler from merging
// them with the plain stores of the other mode.
enum : int { D_ELEM = 0, D_VEC = 1, D_VEC_NT = 2 };
constexpr int CPOL_NT = 2;  // nt
template <typename V>
__device__ inline void store16_nt(const V &v, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, voff, soff, CPOL_NT);
#else
    (void)v, (void)rsrc, (void)voff, (void)soff;
#endif
}
__device__ inline __amdgpu_buffer_rsrc_t d_block_rsrc(const void *origin)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(origin), (short)0, DMA_RANGE, BUFFER_RSRC_WORD3);
}
template <typename E, int WTM, int WTN, typename SO, int NR = WTM>
__device__ inline void store_staged_block(const E *stg, SO stage_off, E *__restrict__ D, int64_t ldd,
                                          int row0, int col0, int M, int N, int dvec, int lane, int r0 = 0)
{
    using V8 = typename Elem<E>::v8;
    constexpr int SCH = WTN / 8;
    constexpr int ROWS_PER_PASS = 64 / SCH;
    constexpr int PASSES = NR / ROWS_PER_PASS;
    static_assert(NR % ROWS_PER_PASS == 0 && NR <= WTM, "whole passes");
    const int rc = lane % SCH, rr = lane / SCH;
    const int col = col0 + 8 * rc;
    if (dvec && row0 + r0 + NR <= M && col0 + WTN <= N) {
        constexpr int BATCH = PASSES < 16 ? PASSES : 16;
        static_assert(PASSES % BATCH == 0, "whole batches");
        E *dst = D + (int64_t)(row0 + r0 + rr) * ldd + col;
        const int64_t pass_stride = (int64_t)ROWS_PER_PASS * ldd;
#pragma unroll
        for (int p0 = 0; p0 < PASSES; p0 += BATCH) {
            V8 v[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
                v[b] = *reinterpret_cast<const V8 *>(stg + stage_off(r0 + (p0 + b) * ROWS_PER_PASS + rr, rc));
            if (dvec == D_VEC_NT) {
                const auto r = d_block_rsrc(D + (int64_t)(row0 + r0) * ldd + col0);
                const uint32_t voff = (uint32_t)(rr * ldd * 2 + 16 * rc);
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    store16_nt(v[b], r, voff, (uint32_t)((p0 + b) * pass_stride * 2));
            } else {
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    *reinterpret_cast<V8 *>(dst + (p0 + b) * pass_stride) = v[b];
            }
        }
        return;
    }
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const int r = r0 + pass * ROWS_PER_PASS + rr;
        const V8 v = *reinterpret_cast<const V8 *>(stg + stage_off(r, rc));
        const int row = row0 + r;
        if (row < M) {
            E *dst = D + (int64_t)row * ldd + col;
            if (dvec && col + 7 < N) {
                *reinterpret_cast<V8 *>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < N)
                        dst[e] = v[e];
            }
        }
    }
}

// Main path for 16-byte aligned operands with K, lda, ldb multiples of 8 and
// in-tile byte offsets below 2^31 (see dma_offsets_fit).
//
// Operand tiles move global → LDS with buffer_load_dwordx4 … lds: one wave
// instruction fills 64 consecutive 16-byte LDS slots (ROWS_PER_DMA whole
// rows), so the swizzle is applied on the source side: lane l fills physical
// chunk l mod RC of row l / RC and fetches the logical chunk stored there.
// Each DMA is a buffer descriptor whose base is the tile origin + k (in
// SGPRs) plus a per-lane 32-bit offset fixed for the whole K loop.  (The
// buffer form, unlike the global form, lets the compiler keep partial
// lgkmcnt waits on the LDS fragment reads.)
//
// Tails: rows of A past M only feed rows of D past M, which are never
// stored (likewise B and N), so such rows are clamped to the last valid row
// instead of being zeroed.  Past K both operands must be exactly zero
// (0·NaN would poison valid outputs): in the last K-tile, lanes whose chunk
// lies beyond K get an offset past the descriptor's range, for which the
// buffer unit returns zeros.
//
// K loop over STAGES LDS stages (a ring, as in the pages' multi-stage
// pipeline, with waits and barriers in place of mbarrier phases):
//   stage kt mod STAGES holds K-tile kt; DMAs for K-tiles kt+1 .. kt+STAGES-1
//   are in flight (the prologue issues K-tiles 0 .. STAGES-1);
//   K-steps 0 .. KSTEPS-2 each read the next step's fragments into the other
//   register buffer while issuing their own MFMAs;
//   wait until K-tile kt+1 has landed (vmcnt), barrier: every wave has
//   finished reading stage kt mod STAGES;
//   the last K-step's MFMAs run from registers while the next stage's K-step
//   0 is read and the drained stage is refilled with K-tile kt+STAGES (past
//   the end: an all-out-of-range DMA, i.e. a no-op that keeps the loop
//   branch-free and the vmcnt bookkeeping uniform).
template <int MF>
struct AccOf {
    typedef f32x16 type;  // 32×32 MFMA: 16 fp32 per lane
};
template <>
struct AccOf<16> {
    typedef f32x4 type;  // 16×16 MFMA: 4 fp32 per lane
};

template <typename E, int BM, int BN, int WM, int WN, int BK_, int STAGES, int OCC, int DMA_STEPS, int KROT,
          int MF = 32>
__global__ __launch_bounds__(WM *WN * 64) TG_WAVES_PER_SIMD(OCC *(WM * WN > 4 ? WM * WN / 4 : 1)) void gemm_dma_kernel(
    const E *__restrict__ A, const E *__restrict__ B, E *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec)
{
    using V8 = typename Elem<E>::v8;
    using V4 = typename Elem<E>::v4;
    using T = OperandTile<BK_>;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    using Acc = typename AccOf<MF>::type;
    constexpr int TM = WTM / MF, TN = WTN / MF;
    constexpr int KW = MF == 32 ? 16 : 32;  // K per MFMA
    constexpr int KSTEPS = BK_ / KW;
    constexpr int CPK = KW / 8;  // 16-byte chunks per row per K-step
    constexpr int ACC_REGS = MF * MF / 64;
    constexpr int A_PASSES = BM / T::ROWS_PER_DMA / NW, B_PASSES = BN / T::ROWS_PER_DMA / NW;
    constexpr int DMA_PER_TILE = A_PASSES + B_PASSES;
    constexpr int STAGE = (BM + BN) * BK_;
    static_assert(MF == 32 || MF == 16, "32×32×16 or 16×16×32 MFMA");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA tile");
    static_assert((BM / T::ROWS_PER_DMA) % NW == 0 && (BN / T::ROWS_PER_DMA) % NW == 0,
                  "DMA row groups must split evenly over the waves");
    static_assert(KSTEPS % 2 == 0, "fragment buffers alternate per K-step");
    static_assert(STAGES >= 2 && STAGES * STAGE * 2 * OCC <= 160 * 1024, "LDS budget");
    // At the wait of iteration kt, K-tiles up to kt+STAGES-1 have been issued;
    // K-tile kt+1 must have landed, so STAGES-2 K-tiles may stay in flight.
    constexpr int VM_IN_FLIGHT = (STAGES - 2) * DMA_PER_TILE;
    static_assert((STAGES - 1) * DMA_PER_TILE <= 63, "vmcnt holds 6 bits");

    __shared__ __attribute__((aligned(1024))) E smem[STAGES * STAGE];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // DMA source of this lane in pass p: tile row t = ROWS_PER_DMA·(p·NW + wave)
    // + lane / RC, whose physical chunk lane mod RC holds logical chunk
    // kc = (lane mod RC) ^ swz(t); byte offset from the tile origin.
    const int dr = lane / T::RC, dpc = lane % T::RC;
    uint32_t a_off[A_PASSES], b_off[B_PASSES];
    int a_kc[A_PASSES], b_kc[B_PASSES];
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        a_kc[p] = dpc ^ T::swz(t);
        a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda * 2 + 16 * a_kc[p]);
    }
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        b_kc[p] = dpc ^ T::swz(t);
        b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb * 2 + 16 * b_kc[p]);
    }
    const char *a_tile = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_tile = reinterpret_cast<const char *>(B + (int64_t)n0 * ldb);
    const int KT = (K + BK_ - 1) / BK_;

    struct DmaTile {
        __amdgpu_buffer_rsrc_t ra, rb;
        E *as, *bs;
        int klim;  // valid K elements in this K-tile (0 past the end)
    };
    // K-tile order: this workgroup starts at K-tile krot and wraps around.
    // With KROT the eight XCDs (workgroup w runs on XCD w mod 8) start at
    // K offsets spread evenly over the row, so that at any moment the XCDs
    // stream from different address ranges of B instead of all requesting
    // the same column band of every row; a streaming (HBM-bound) launch
    // gains about a quarter of its bandwidth.  Only the order of the K
    // summation changes.
    const int krot = KROT && KT > 0 ? (int)(blockIdx.x % 8) * KT / 8 : 0;
    auto dma_tile = [&](int kt) {
        int pk = kt + krot;
        if (pk >= KT)
            pk -= KT;
        const int k = pk * BK_;
        DmaTile d;
        d.ra = __builtin_amdgcn_make_buffer_rsrc((void *)(a_tile + 2 * k), (short)0, DMA_RANGE,
                                                 BUFFER_RSRC_WORD3);
        d.rb = __builtin_amdgcn_make_buffer_rsrc((void *)(b_tile + 2 * k), (short)0, DMA_RANGE,
                                                 BUFFER_RSRC_WORD3);
        d.as = smem + (kt % STAGES) * STAGE;
        d.bs = d.as + BM * BK_;
        d.klim = kt < KT ? K - k : 0;
        return d;
    };
    // i-th DMA of a K-tile: A passes first, then B passes
    auto dma_pass = [&](const DmaTile &d, int i) {
        if (i < A_PASSES)
            dma16<CPOL_CACHED>(d.ra, d.as + (i * NW + wave) * T::ROWS_PER_DMA * BK_,
                  8 * a_kc[i] < d.klim ? a_off[i] : DMA_OOB);
        else
            dma16<KROT ? CPOL_STREAM : CPOL_CACHED>(
                d.rb, d.bs + ((i - A_PASSES) * NW + wave) * T::ROWS_PER_DMA * BK_,
                  8 * b_kc[i - A_PASSES] < d.klim ? b_off[i - A_PASSES] : DMA_OOB);
    };

    const int frag_row = MF == 32 ? frag_row_of(lane) : frag16_row_of(lane);
    const int frag_hi = MF == 32 ? frag_hi_of(lane) : frag16_hi_of(lane);
    V8 fa[2][TM], fb[2][TN];
    // one fragment of K-step kk of the K-tile in stage s: q < TM is A
    // fragment q, else B fragment q - TM
    auto read_frag = [&](int s, int kk, int q, V8 *a, V8 *b) {
        const E *as = smem + s * STAGE;
        const E *bs = as + BM * BK_;
        const int c = kk * CPK + frag_hi;
        if (q < TM)
            a[q] = *reinterpret_cast<const V8 *>(as + T::off(wm * WTM + q * MF + frag_row, c));
        else
            b[q - TM] = *reinterpret_cast<const V8 *>(
                bs + T::off(wn * WTN + (q - TM) * MF + frag_row, c));
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < ACC_REGS; ++v)
                acc[i][j][v] = 0.0f;

    // One K-step's TM·TN MFMAs on fragments (a, b), with the companion work
    // pinned between them in program order (sched_barrier fences each slot):
    // after MFMA i comes the next K-step's LDS read i (for i < TM+TN, in the
    // order the next step first uses them: A0, B0..B(TN-1), A1..A(TM-1)) and,
    // when `dma` is given, DMA pass i.  The matrix core runs each MFMA while
    // the wave issues the companions; fewer than 16 LDS reads are ever in
    // flight, so the compiler's lgkmcnt waits stay partial.
    constexpr int NFRAG = TM + TN;
    constexpr int SLOTS = TM * TN;
    auto frag_of_slot = [](int i) { return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN; };
    // DMA passes [lo, hi) of `dma` ride along from slot 1 on, one every
    // `every` slots, so they spread evenly over the step (between and beside
    // the fragment reads) instead of arriving at the memory pipe in a burst;
    // passes that outnumber the slots go after the last MFMA.
    auto step = [&](const V8 *a, const V8 *b, bool with_reads, int rs, int rkk, V8 *na,
                    V8 *nb, const DmaTile *dma, int lo, int hi, int every) {
        constexpr int first = 1;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int ti = i / TN, tj = i % TN;
            acc[ti][tj] = Elem<E>::mfma(b[tj], a[ti], acc[ti][tj]);
            MFMA_FIRST();
            if (with_reads && i < NFRAG)
                read_frag(rs, rkk, frag_of_slot(i), na, nb);
            if (dma && i >= first && (i - first) % every == 0 && lo + (i - first) / every < hi)
                dma_pass(*dma, lo + (i - first) / every);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = SLOTS; i < NFRAG; ++i)  // reads left when fragments outnumber slots
            if (with_reads)
                read_frag(rs, rkk, frag_of_slot(i), na, nb);
        if (dma)  // DMA passes left when they outnumber the slots
            for (int p = lo + (SLOTS - first + every - 1) / every; p < hi; ++p)
                dma_pass(*dma, p);
    };

    // DMA schedule.  The refill of the stage drained at a barrier is spread
    // over DMA_STEPS K-steps: the first P1 passes in the post-barrier step,
    // the rest in the next iteration's first DMA_STEPS-1 leading steps.  The
    // memory pipe (64 bytes per clock per CU, i.e. 16 clocks per 1 KiB DMA)
    // then sees an even trickle instead of a burst that backs up and stalls
    // the waves' in-order instruction streams, MFMAs included; the price is
    // a shorter latency budget for the last passes (they must land by the
    // wait at the end of the leading steps when STAGES == 2).
    constexpr int DSTEPS = DMA_STEPS < 1 ? 1 : DMA_STEPS > KSTEPS ? KSTEPS : DMA_STEPS;
    constexpr bool SPREAD = DSTEPS > 1;
    constexpr int P1 = (DMA_PER_TILE + DSTEPS - 1) / DSTEPS;
    constexpr int DMA_SLOTS = SLOTS;
    constexpr int EVERY_POST = DMA_SLOTS / P1 > 0 ? DMA_SLOTS / P1 : 1;
    constexpr int REST = DMA_PER_TILE - P1;
    constexpr int REST_PER_STEP = SPREAD ? (REST + DSTEPS - 2) / (DSTEPS - 1) : 0;
    constexpr int EVERY_LEAD =
        REST_PER_STEP > 0 && DMA_SLOTS / REST_PER_STEP > 0 ? DMA_SLOTS / REST_PER_STEP : 1;
    // outstanding DMA passes allowed at the prologue wait (K-tile 0 landed)
    constexpr int VM_PROLOGUE = (STAGES - 2) * DMA_PER_TILE + P1;
    static_assert(VM_PROLOGUE <= 63, "vmcnt holds 6 bits");

    // prologue: K-tiles 0 .. STAGES-1 (with spreading, only the first P1
    // passes of K-tile STAGES-1; iteration 0 issues the rest); wait for K-tile 0
#pragma unroll
    for (int t = 0; t < STAGES; ++t) {
        const DmaTile d = dma_tile(t);
#pragma unroll
        for (int i = 0; i < DMA_PER_TILE; ++i)
            if (!SPREAD || t < STAGES - 1 || i < P1)
                dma_pass(d, i);
    }
    wait_vmem<VM_PROLOGUE>();
    barrier_lds();
#pragma unroll
    for (int q = 0; q < NFRAG; ++q)
        read_frag(0, 0, q, fa[0], fb[0]);

    // K-steps 0 .. KSTEPS-2 of the K-tile in stage s, each reading the next
    // step's fragments (the last step's fragments end up in buffer 1) and,
    // with spreading, carrying the remaining passes of K-tile dkt
    auto leading_steps = [&](int s, int dkt) {
        const DmaTile d = dma_tile(dkt);
#pragma unroll
        for (int kk = 0; kk < KSTEPS - 1; ++kk) {
            const int lo = P1 + kk * REST_PER_STEP;
            const int hi = lo + REST_PER_STEP < DMA_PER_TILE ? lo + REST_PER_STEP : DMA_PER_TILE;
            step(fa[kk & 1], fb[kk & 1], true, s, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1],
                 SPREAD && kk < DSTEPS - 1 ? &d : nullptr, lo, hi, EVERY_LEAD);
        }
    };
    // steady state: a next K-tile exists (the last one is peeled off so the
    // loop body is straight-line)
    for (int kt = 0; kt < KT - 1; ++kt) {
        const int s = kt % STAGES;
        leading_steps(s, kt + STAGES - 1);
        wait_vmem<VM_IN_FLIGHT>();  // K-tile kt+1 has landed (this wave's part)
        barrier_lds();              // ... for every wave; stage s is drained
        const DmaTile d = dma_tile(kt + STAGES);
        step(fa[1], fb[1], true, (kt + 1) % STAGES, 0, fa[0], fb[0], &d, 0, P1, EVERY_POST);
    }
    // the last K-tile (with 16×16 MFMAs without a branch: a conditional tail
    // makes the register allocator rotate accumulators; with K = 0 it reads
    // stage 0, which the prologue filled with zeros — every DMA there read
    // past the range — so it adds nothing)
    if (MF == 16 || KT > 0) {
        leading_steps(KT > 0 ? (KT - 1) % STAGES : 0, KT - 1 + STAGES - 1);
        step(fa[1], fb[1], false, 0, 0, fa[0], fb[0], nullptr, 0, 0, 1);
    }
    wait_vmem<0>();  // no LDS DMA may be outstanding when the wave ends

    // Epilogue, staged through LDS so that global stores are whole lines.
    // Accumulator register v of lane l holds D row (l % 32) and D column
    // 8·(v/4) + 4·(l/32) + v%4 of its 32×32 tile.  After a barrier (every wave
    // is done with the operand stages) each wave writes its WTM×WTN block as
    // fp16 into its own region of the stage memory — row-major, 16-byte chunk
    // index XORed with the row so the 32 rows one write instruction touches
    // spread over the banks — then reads it back 16 bytes per lane along rows
    // and stores those: each store instruction writes 64·16 bytes as
    // contiguous row segments.  Conversion is fp32 → fp16 round-to-nearest-even.
    static_assert(NW * WTM * WTN * 2 <= STAGES * STAGE * 2, "staging fits in the stage memory");
    constexpr int SROW = WTN;                 // staging row length (elements)
    constexpr int SCH = WTN / 8;              // 16-byte chunks per staging row
    static_assert((SCH & (SCH - 1)) == 0 && SCH >= 2, "chunk swizzle needs a power of two");
    auto stage_off = [](int r, int chunk) { return r * SROW + ((chunk ^ (r & (SCH - 1))) << 3); };
    barrier_lds();
    E *stg = smem + wave * WTM * WTN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < ACC_REGS / 4; ++g) {
                V4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (E)acc[i][j][g * 4 + r];  // round to nearest even
                // four consecutive D columns of row r
                const int r = i * MF + frag_row;
                const int c = j * MF + (MF == 32 ? g * 8 + frag_hi * 4 : frag_hi * 4);
                *reinterpret_cast<V4 *>(stg + stage_off(r, c / 8) + (c & 7)) = h;
            }
    store_staged_block<E, WTM, WTN>(stg, stage_off, D, ldd, m0 + wm * WTM, n0 + wn * WTN, M, N, dvec, lane);
}

// Producer/consumer form of the 128×128 tile ("TIRx 与高性能GEMM (上)":
// the closing summary names the producer/consumer split as the step after
// the multi-stage pipeline — warp specialization).  Eight waves, two per
// SIMD: waves 0..3 are consumers (a 2×2 grid of 64×64 blocks of D, 16×16×32
// MFMAs on 64 accumulators each, fragment reads from LDS), waves 4..7 are
// producers (every operand DMA of the tile, nothing else).  A DMA that
// stalls at issue — the memory pipeline backed up behind L2 misses — then
// stalls only its producer wave, while the consumer on the same SIMD keeps
// issuing MFMAs.  On CDNA all waves of a workgroup get the same register
// allocation, so the split fits where a consumer needs at most half the
// register file: here, not at 256×256.
//
// STAGES LDS stages of 32 KiB (A's and B's 128 rows of one 64-K tile, the
// same swizzle and source-side DMA addressing as the other kernels).  One
// workgroup barrier per K-tile, in the middle of the consumers' K-tile t:
// before it the producers wait until K-tile t+1 has landed and the
// consumers finish reading stage t; after it the producers refill stage t
// with K-tile t+STAGES.  A partial K-tile is the first one (its columns
// below 0 read as zero); K-tiles past the end get empty ranges.  A last
// barrier after the producers' final wait frees all stages for the
// consumers' staged epilogue.
template <typename E, int STAGES>
__global__ __launch_bounds__(512) TG_WAVES_PER_SIMD(2) void gemm_ws_kernel(
    const E *__restrict__ A, const E *__restrict__ B, E *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec)
{
    using V8 = typename Elem<E>::v8;
    using V4 = typename Elem<E>::v4;
    constexpr int BM = 128, BN = 128, BK_ = 64, MF = 16;
    using T = OperandTile<BK_>;
    constexpr int NC = 4;                       // consumer waves (and producer waves)
    constexpr int WTM = 64, WTN = 64;           // consumer block
    constexpr int TM = WTM / MF, TN = WTN / MF;
    constexpr int CPK = 4;
    constexpr int PIECE = T::ROWS_PER_DMA * BK_;               // elements one DMA fills (1 KiB)
    constexpr int PASSES = BM / T::ROWS_PER_DMA / NC;          // DMAs per producer per operand K-tile
    constexpr int DPT = 2 * PASSES;                            // DMAs per producer per K-tile
    constexpr int STAGE = (BM + BN) * BK_;
    static_assert(STAGES >= 3 && STAGES * STAGE * 2 <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 1) * DPT <= 63, "vmcnt holds 6 bits");
    static_assert(NC * WTM * WTN <= STAGE * STAGES, "staging fits");

    __shared__ __attribute__((aligned(1024))) E smem[STAGES * STAGE];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KT = (K + BK_ - 1) / BK_;
    const int k0 = K - BK_ * KT;  // <= 0: the first K-tile may be partial

    if (wave >= NC) {
        // ---------------- producer: DMA pieces 4p + pw of A and of B
        const int pw = wave - NC;
        const int dr = lane / T::RC;
        static_assert((NC * T::ROWS_PER_DMA) % 16 == 0, "swizzle repeats per pass");
        const int kc = (lane % T::RC) ^ T::swz(T::ROWS_PER_DMA * pw + dr);
        uint32_t a_off[PASSES], b_off[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int t = T::ROWS_PER_DMA * (p * NC + pw) + dr;
            a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda * 2 + 16 * kc);
            b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb * 2 + 16 * kc);
        }
        const char *a_tile = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
        const char *b_tile = reinterpret_cast<const char *>(B + (int64_t)n0 * ldb);
        auto issue = [&](int t, bool first) {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a_tile + 2 * (int64_t)(k0 + t * BK_)), (short)0, t < KT ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(b_tile + 2 * (int64_t)(k0 + t * BK_)), (short)0, t < KT ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
            E *st = smem + (t % STAGES) * STAGE;
            const bool neg = first && k0 + 8 * kc < 0;  // columns below 0 of the partial first K-tile
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                dma16<CPOL_CACHED>(ra, st + (p * NC + pw) * PIECE, neg ? DMA_OOB : a_off[p]);
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                dma16<CPOL_CACHED>(rb, st + BM * BK_ + (p * NC + pw) * PIECE, neg ? DMA_OOB : b_off[p]);
        };
        issue(0, true);
#pragma unroll
        for (int t = 1; t < STAGES; ++t)
            issue(t, false);
        wait_vmem<(STAGES - 1) * DPT>();  // K-tile 0 has landed
        barrier_lds();  // (not __syncthreads: that would wait for every DMA in flight)
        for (int t = 0; t < KT; ++t) {
            wait_vmem<(STAGES - 2) * DPT>();  // K-tile t+1 has landed
            barrier_lds();                   // consumers are done with stage t
            issue(t + STAGES, false);
        }
        wait_vmem<0>();
        barrier_lds();  // every stage is free for the epilogue
        return;
    }

    // ---------------- consumer
    const int wm = wave / 2, wn = wave % 2;
    const int frag_row = frag16_row_of(lane), frag_hi = frag16_hi_of(lane);
    int a_lane[2], b_lane[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        a_lane[kk] = T::off(wm * WTM + frag_row, kk * CPK + frag_hi);
        b_lane[kk] = BM * BK_ + T::off(wn * WTN + frag_row, kk * CPK + frag_hi);
    }
    static_assert(T::swz(16) == T::swz(0), "swizzle period");
    V8 fa[2][TM], fb[2][TN];
    auto read_frag = [&](int s, int kk, int q, V8 *a, V8 *b) {
        const E *st = smem + s * STAGE;
        if (q < TM)
            a[q] = *reinterpret_cast<const V8 *>(st + a_lane[kk] + q * MF * BK_);
        else
            b[q - TM] = *reinterpret_cast<const V8 *>(st + b_lane[kk] + (q - TM) * MF * BK_);
    };
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int NFRAG = TM + TN, SLOTS = TM * TN, RS = SLOTS / NFRAG;
    static_assert(RS >= 1, "reads fit the slots");
    auto frag_of_slot = [](int i) { return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN; };
    auto step = [&](const V8 *a, const V8 *b, int rs, int rkk, V8 *na, V8 *nb) {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            acc[i / TN][i % TN] = Elem<E>::mfma(b[i % TN], a[i / TN], acc[i / TN][i % TN]);
            MFMA_FIRST();
            if (i % RS == 0 && i / RS < NFRAG)
                read_frag(rs, rkk, frag_of_slot(i / RS), na, nb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    barrier_lds();  // K-tile 0 has landed
#pragma unroll
    for (int q = 0; q < NFRAG; ++q)
        read_frag(0, 0, q, fa[0], fb[0]);
    int s = 0;
    for (int t = 0; t < KT; ++t) {
        step(fa[0], fb[0], s, 1, fa[1], fb[1]);
        barrier_lds();  // this K-tile's stage is read; K-tile t+1 has landed
        const int s1 = s + 1 == STAGES ? 0 : s + 1;
        step(fa[1], fb[1], s1, 0, fa[0], fb[0]);  // (past the last K-tile the reads are unused)
        s = s1;
    }
    barrier_lds();  // the producers' last DMAs have landed: every stage is free

    // staged epilogue: each consumer stages its 64×64 block in its own 8 KiB
    constexpr int SROW = WTN, SCH = WTN / 8;
    auto stage_off = [](int r, int chunk) { return r * SROW + ((chunk ^ (r & (SCH - 1))) << 3); };
    E *stg = smem + wave * WTM * WTN;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            V4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = (E)acc[i][j][r];  // round to nearest even
            const int r = i * MF + frag_row;
            const int c = j * MF + frag_hi * 4;
            *reinterpret_cast<V4 *>(stg + stage_off(r, c / 8) + (c & 7)) = h;
        }
        store_staged_block<E, WTM, WTN, decltype(stage_off), MF>(stg, stage_off, D, ldd, m0 + wm * WTM,
                                                                 n0 + wn * WTN, M, N, dvec, lane, i * MF);
    }
}

// Variant of gemm_dma_kernel for the largest tile with separate LDS rings
// for the two operands: three stages of A and two of B (BK = 64: 3·32 + 2·32
// KiB = 160 KiB for 256×256).  With one ring of two stages the refill of a
// drained stage has one K-tile to land, so its 16 DMAs per wave had to be
// packed into two of the four K-steps, where they saturate the CU's address
// unit (64 bytes per clock) and stall the wave's in-order issue behind it,
// MFMAs included.  The third A stage gives A's refill two K-tiles, so each of
// the four K-steps now carries four DMAs per wave: B's refill in the last
// K-step of a tile and the first of the next (same latency budget as before),
// A's refill, one K-tile further ahead, in the next two.  Per iteration t
// with MF = 32 (four 16-K steps of 32×32×16 MFMAs):
//   K-step 0: B(t+1), second half      K-step 1: A(t+2), first half
//   K-step 2: A(t+2), second half      wait until all but A(t+2) landed
//   barrier (A stage t mod 3 and B stage t mod 2 are drained)
//   K-step 3: B(t+2), first half (and the fragments of K-tile t+1, step 0)
// With MF = 16 (two 32-K steps of 64 16×16×32 MFMAs each) K-step 0 carries
// all of A(t+2), then the wait and the barrier, and K-step 1 all of B(t+2),
// one DMA every eighth MFMA.  Everything else (swizzle, fragment reads, staged epilogue) is as in
// gemm_dma_kernel; rows past M or N are clamped, and a K that is not a
// multiple of 64 makes the first K-tile (not the last) the partial one.
template <typename E, int BM, int BN, int WM, int WN, int MF>
__global__ __launch_bounds__(WM *WN * 64) TG_WAVES_PER_SIMD(1) void gemm_dma3_kernel(
    const E *__restrict__ A, const E *__restrict__ B, E *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec)
{
    using V8 = typename Elem<E>::v8;
    using V4 = typename Elem<E>::v4;
    constexpr int BK_ = 64, SA = 3, SB = 2;
    using T = OperandTile<BK_>;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    using Acc = typename AccOf<MF>::type;
    constexpr int TM = WTM / MF, TN = WTN / MF;
    constexpr int KW = MF == 32 ? 16 : 32;  // K per MFMA
    constexpr int KSTEPS = BK_ / KW;
    constexpr int CPK = KW / 8;  // 16-byte chunks per row per K-step
    constexpr int ACC_REGS = MF * MF / 64;
    constexpr int A_PASSES = BM / T::ROWS_PER_DMA / NW, B_PASSES = BN / T::ROWS_PER_DMA / NW;
    constexpr int AH = A_PASSES / 2, BH = B_PASSES / 2;
    constexpr int STAGE_A = BM * BK_, STAGE_B = BN * BK_;
    static_assert(MF == 32 || MF == 16, "32×32×16 or 16×16×32 MFMA");
    static_assert(A_PASSES % 2 == 0 && B_PASSES % 2 == 0, "DMA passes split in halves");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA tile");
    static_assert((BM / T::ROWS_PER_DMA) % NW == 0 && (BN / T::ROWS_PER_DMA) % NW == 0,
                  "DMA row groups must split evenly over the waves");
    static_assert((SA * STAGE_A + SB * STAGE_B) * 2 <= 160 * 1024, "LDS budget");
    static_assert(A_PASSES + BH + A_PASSES <= 63, "vmcnt holds 6 bits");

    __shared__ __attribute__((aligned(1024))) E smem[SA * STAGE_A + SB * STAGE_B];
    E *const a_ring = smem;
    E *const b_ring = smem + SA * STAGE_A;

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int dr = lane / T::RC, dpc = lane % T::RC;
    uint32_t a_off[A_PASSES], b_off[B_PASSES];
    int a_kc[A_PASSES], b_kc[B_PASSES];
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        a_kc[p] = dpc ^ T::swz(t);
        a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda * 2 + 16 * a_kc[p]);
    }
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        b_kc[p] = dpc ^ T::swz(t);
        b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb * 2 + 16 * b_kc[p]);
    }
    const char *a_tile = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_tile = reinterpret_cast<const char *>(B + (int64_t)n0 * ldb);
    const int KT = (K + BK_ - 1) / BK_;
    // K-tile t covers columns k0 + 64t .. k0 + 64t + 63 with k0 = K - 64·KT
    // (<= 0): only the first K-tile can be partial, and its columns below 0
    // read as zero (those lanes get an offset past the range), so the DMAs
    // of the K loop carry no per-lane bounds test (a vector select per DMA
    // costs the matrix core issue cycles); K-tiles past the last get an
    // empty buffer range, where every lane reads zero.
    const int k0 = K - BK_ * KT;

    // DMA source and LDS stage of one operand's K-tile
    struct Op {
        __amdgpu_buffer_rsrc_t r;
        E *dst;
    };
    auto op_a = [&](int t) {
        Op o;
        o.r = __builtin_amdgcn_make_buffer_rsrc((void *)(a_tile + 2 * (int64_t)(k0 + t * BK_)), (short)0,
                                                t < KT ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
        o.dst = a_ring + (t % SA) * STAGE_A;
        return o;
    };
    auto op_b = [&](int t) {
        Op o;
        o.r = __builtin_amdgcn_make_buffer_rsrc((void *)(b_tile + 2 * (int64_t)(k0 + t * BK_)), (short)0,
                                                t < KT ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
        o.dst = b_ring + (t % SB) * STAGE_B;
        return o;
    };
    auto dma_a = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BK_, a_off[p]);
    };
    auto dma_b = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BK_, b_off[p]);
    };
    // K-tile 0: lanes whose chunk lies below column 0 read zero
    auto dma_a0 = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BK_,
                           k0 + 8 * a_kc[p] >= 0 ? a_off[p] : DMA_OOB);
    };
    auto dma_b0 = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BK_,
                           k0 + 8 * b_kc[p] >= 0 ? b_off[p] : DMA_OOB);
    };

    const int frag_row = MF == 32 ? frag_row_of(lane) : frag16_row_of(lane);
    const int frag_hi = MF == 32 ? frag_hi_of(lane) : frag16_hi_of(lane);
    V8 fa[2][TM], fb[2][TN];
    // The swizzle repeats every 16 rows, so a lane's chunk position in
    // K-step kk is the same for every fragment: one per-lane offset per
    // K-step, and fragment q sits a constant 32 rows further (an immediate
    // offset of the LDS read, no address arithmetic per read).
    static_assert(T::swz(16) == T::swz(0) && WTM % 16 == 0 && WTN % 16 == 0, "swizzle period");
    int a_lane[KSTEPS], b_lane[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        a_lane[kk] = T::off(wm * WTM + frag_row, kk * CPK + frag_hi);
        b_lane[kk] = T::off(wn * WTN + frag_row, kk * CPK + frag_hi);
    }
    // fragment q of K-step kk of the K-tile in A stage sa / B stage sb
    auto read_frag = [&](int sa, int sb, int kk, int q, V8 *a, V8 *b) {
        if (q < TM)
            a[q] = *reinterpret_cast<const V8 *>(a_ring + sa * STAGE_A + a_lane[kk] + q * MF * BK_);
        else
            b[q - TM] = *reinterpret_cast<const V8 *>(b_ring + sb * STAGE_B + b_lane[kk] + (q - TM) * MF * BK_);
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < ACC_REGS; ++v)
                acc[i][j][v] = 0.0f;

    constexpr int NFRAG = TM + TN;
    constexpr int SLOTS = TM * TN;
    // fragment reads every other slot, DMAs in the odd slots between them:
    // the LDS sees reads and DMA writes interleaved rather than in bursts
    constexpr int RSTRIDE = SLOTS / NFRAG;
    static_assert(RSTRIDE >= 2 && RSTRIDE % 2 == 0, "reads go in even slots");
    auto frag_of_slot = [](int i) { return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN; };
    // One K-step: MFMA per slot; the next step's read i after MFMA i (i <
    // NFRAG); the DMA passes [lo, hi) of `o` (A when is_a) from slot 1 at an
    // even stride; passes that outnumber the slots go after the last MFMA.
    auto step = [&](const V8 *a, const V8 *b, bool with_reads, int rsa, int rsb, int rkk,
                    V8 *na, V8 *nb, const Op *o, bool is_a, int lo, int hi) {
        const int n = hi - lo;
        const int every = n > 0 && SLOTS / n > 0 ? SLOTS / n : 1;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int ti = i / TN, tj = i % TN;
            acc[ti][tj] = Elem<E>::mfma(b[tj], a[ti], acc[ti][tj]);
            MFMA_FIRST();
            if (with_reads && i % RSTRIDE == 0 && i / RSTRIDE < NFRAG)
                read_frag(rsa, rsb, rkk, frag_of_slot(i / RSTRIDE), na, nb);
            if (o && i >= 1 && (i - 1) % every == 0 && lo + (i - 1) / every < hi) {
                if (is_a)
                    dma_a(*o, lo + (i - 1) / every);
                else
                    dma_b(*o, lo + (i - 1) / every);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = (SLOTS + RSTRIDE - 1) / RSTRIDE; q < NFRAG; ++q)
            if (with_reads)
                read_frag(rsa, rsb, rkk, frag_of_slot(q), na, nb);
        if (o)
            for (int p = lo + (SLOTS - 1 + every - 1) / every; p < hi; ++p) {
                if (is_a)
                    dma_a(*o, p);
                else
                    dma_b(*o, p);
            }
    };

    if constexpr (KSTEPS == 4) {
        // prologue: A(0), B(0), A(1), first half of B(1); wait for A(0) and B(0)
        {
            const Op a0 = op_a(0), b0 = op_b(0), a1 = op_a(1), b1 = op_b(1);
#pragma unroll
            for (int p = 0; p < A_PASSES; ++p)
                dma_a0(a0, p);
#pragma unroll
            for (int p = 0; p < B_PASSES; ++p)
                dma_b0(b0, p);
#pragma unroll
            for (int p = 0; p < A_PASSES; ++p)
                dma_a(a1, p);
#pragma unroll
            for (int p = 0; p < BH; ++p)
                dma_b(b1, p);
        }
        wait_vmem<A_PASSES + BH>();
        barrier_lds();
#pragma unroll
        for (int q = 0; q < NFRAG; ++q)
            read_frag(0, 0, 0, q, fa[0], fb[0]);

        int sa = 0, sb = 0;  // stages of K-tile kt
        for (int kt = 0; kt < KT - 1; ++kt) {
            const Op bn = op_b(kt + 1), an = op_a(kt + 2);
            step(fa[0], fb[0], true, sa, sb, 1, fa[1], fb[1], &bn, false, BH, B_PASSES);
            step(fa[1], fb[1], true, sa, sb, 2, fa[0], fb[0], &an, true, 0, AH);
            step(fa[0], fb[0], true, sa, sb, 3, fa[1], fb[1], &an, true, AH, A_PASSES);
            wait_vmem<A_PASSES>();  // K-tile kt+1 has landed (this wave's part); A(kt+2) may not
            barrier_lds();          // ... for every wave; A stage sa and B stage sb are drained
            const Op b2 = op_b(kt + 2);
            const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb + 1 == SB ? 0 : sb + 1;
            step(fa[1], fb[1], true, sa1, sb1, 0, fa[0], fb[0], &b2, false, 0, BH);
            sa = sa1;
            sb = sb1;
        }
        if (KT > 0) {
            step(fa[0], fb[0], true, sa, sb, 1, fa[1], fb[1], nullptr, false, 0, 0);
            step(fa[1], fb[1], true, sa, sb, 2, fa[0], fb[0], nullptr, false, 0, 0);
            step(fa[0], fb[0], true, sa, sb, 3, fa[1], fb[1], nullptr, false, 0, 0);
            step(fa[1], fb[1], false, 0, 0, 0, fa[0], fb[0], nullptr, false, 0, 0);
        }
    } else {
        // Two K-steps per K-tile (16×16×32): K-step 0 carries A(t+2), the
        // wait and barrier follow, and K-step 1 carries B(t+2) while it reads
        // the first K-step of tile t+1.  B(t+2) lands in B stage t mod 2,
        // drained at this barrier; A(t+2) in A stage (t-1) mod 3, drained at
        // the previous one.  The prologue issues A(0), B(0), A(1), B(1).
        {
            const Op a0 = op_a(0), b0 = op_b(0), a1 = op_a(1), b1 = op_b(1);
#pragma unroll
            for (int p = 0; p < A_PASSES; ++p)
                dma_a0(a0, p);
#pragma unroll
            for (int p = 0; p < B_PASSES; ++p)
                dma_b0(b0, p);
#pragma unroll
            for (int p = 0; p < A_PASSES; ++p)
                dma_a(a1, p);
#pragma unroll
            for (int p = 0; p < B_PASSES; ++p)
                dma_b(b1, p);
        }
        wait_vmem<A_PASSES + B_PASSES>();
        barrier_lds();
#pragma unroll
        for (int q = 0; q < NFRAG; ++q)
            read_frag(0, 0, 0, q, fa[0], fb[0]);

        int sa = 0, sb = 0;
        for (int kt = 0; kt < KT - 1; ++kt) {
            const Op an = op_a(kt + 2);
            step(fa[0], fb[0], true, sa, sb, 1, fa[1], fb[1], &an, true, 0, A_PASSES);
            wait_vmem<A_PASSES>();  // B(kt+1) and A(kt+1) have landed; A(kt+2) may not
            barrier_lds();
            const Op b2 = op_b(kt + 2);
            const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb + 1 == SB ? 0 : sb + 1;
            step(fa[1], fb[1], true, sa1, sb1, 0, fa[0], fb[0], &b2, false, 0, B_PASSES);
            sa = sa1;
            sb = sb1;
        }
        // the last K-tile; with K = 0 every DMA above had an empty range, so
        // the stages hold zeros and this adds nothing (no branch here: a
        // conditional tail made the register allocator rotate accumulators)
        step(fa[0], fb[0], true, sa, sb, 1, fa[1], fb[1], nullptr, false, 0, 0);
        step(fa[1], fb[1], false, 0, 0, 0, fa[0], fb[0], nullptr, false, 0, 0);
    }
    wait_vmem<0>();  // no LDS DMA may be outstanding when the wave ends

    // staged epilogue, as in gemm_dma_kernel
    static_assert(NW * WTM * WTN <= SA * STAGE_A + SB * STAGE_B, "staging fits in the stage memory");
    constexpr int SROW = WTN;
    constexpr int SCH = WTN / 8;
    static_assert((SCH & (SCH - 1)) == 0 && SCH >= 2, "chunk swizzle needs a power of two");
    auto stage_off = [](int r, int chunk) { return r * SROW + ((chunk ^ (r & (SCH - 1))) << 3); };
    barrier_lds();
    E *stg = smem + wave * WTM * WTN;
    static_assert(TM % 4 == 0, "quarters of whole fragment rows");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int i = q * TM / 4; i < (q + 1) * TM / 4; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < ACC_REGS / 4; ++g) {
                    V4 h;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        h[r] = (E)acc[i][j][g * 4 + r];  // round to nearest even
                    // four consecutive D columns of row r
                    const int r = i * MF + frag_row;
                    const int c = j * MF + (MF == 32 ? g * 8 + frag_hi * 4 : frag_hi * 4);
                    *reinterpret_cast<V4 *>(stg + stage_off(r, c / 8) + (c & 7)) = h;
                }
        store_staged_block<E, WTM, WTN, decltype(stage_off), WTM / 4>(stg, stage_off, D, ldd, m0 + wm * WTM,
                                                                      n0 + wn * WTN, M, N, dvec, lane,
                                                                      q * WTM / 4);
    }
}

// Persistent form of the 256×256 kernel (the pages' Step 6: a fixed pool of
// workgroups, each taking tile after tile — "TIRx 与高性能GEMM (上)",
// section "Step 6：Persistent kernel 让 CTA 持续领取 tile").  One workgroup
// per compute unit (the grid is a multiple of 8, so workgroup w stays on XCD
// w mod 8); workgroup w takes the tiles of virtual ids w, w + P, w + 2P, ...
// (P = grid size) through the same XCD-grouped order as the one-tile-per-
// workgroup launch, so the tiles resident on an XCD at any moment are the
// same ones.  K must be a multiple of 64 and at least 128 (no partial
// K-tile; the next tile's first two K-tiles load during the last two).
//
// The K-tiles of a workgroup's tiles form one stream: the refills run two
// K-tiles ahead of the matrix cores across tile boundaries, so the next
// tile's first operand tiles are already landing while the current tile's
// last K-tiles are multiplied, and no tile starts by waiting for its first
// loads.  Rings: SA_ stages of A and 5 - SA_ of B (32 KiB each); the operand
// with three stages is refilled in K-step 0 (two K-tiles of latency budget),
// the other in K-step 1, after the barrier that drains its stage.
//
// Epilogue, at the last K-tile of a tile, with no workgroup barrier: the
// 3-stage operand's stage of that K-tile is drained at that K-tile's
// barrier and refilled only in the next tile's first K-step, so it holds
// the staging of D (32 KiB), while the other operand's refill goes out in
// that K-tile as in every other one (its data has the whole epilogue to
// land).  Each wave stages its 128×128 block in four 32-row quarters of 8
// KiB, in exactly the eight 1 KiB pieces of that stage that its own DMAs
// fill (a DMA instruction of wave w writes the piece 4p + w of a stage), so
// the only later writers of its staging memory are its own DMAs, issued
// after its own staging reads have completed.  Per quarter: fp32 → element
// RNE into LDS (16-byte chunk index XORed with the row), read back 16 bytes
// per lane along rows, store whole row segments; the accumulators are
// cleared as they are read.  Then the next tile's first K-step runs on
// fragments read before the epilogue.  The wave waits for all its DMAs
// before its first store, so the next tile's first K-tile needs no wait
// and the stores drain behind it.
//
// RS0: fragment reads of K-step 0 every RS0-th MFMA slot (2: in the first
// half of the step, so they have landed by the barrier's wait; 4: spread).
//
// STAMP (measurement only, tg_gemm_f16_xcd_stamps): the same kernel, plus
// three words per workgroup in `stamps` — the constant 100 MHz clock when it
// starts and when all its waves are done, and the XCD it ran on.  The GEMM
// launch passes a null `stamps` and never reads it.
template <typename E, int SA_, int GM, int RS0, bool STAMP = false>
__global__ __launch_bounds__(256) TG_WAVES_PER_SIMD(1) void gemm_pers_kernel(
    const E *__restrict__ A, const E *__restrict__ B, E *__restrict__ D,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, int tiles_m, int tiles_n,
    int dvec, unsigned long long *__restrict__ stamps)
{
    if constexpr (STAMP) {
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        unsigned xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        if (threadIdx.x == 0) {
            stamps[3 * blockIdx.x] = t0;
            stamps[3 * blockIdx.x + 2] = xcc;
        }
    }
    using V8 = typename Elem<E>::v8;
    using V4 = typename Elem<E>::v4;
    constexpr int BM = 256, BN = 256, WM = 2, WN = 2, MF = 16, BK_ = 64;
    constexpr int SA = SA_, SB = 5 - SA_;
    static_assert(SA == 2 || SA == 3, "three stages of one operand, two of the other");
    using T = OperandTile<BK_>;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / MF, TN = WTN / MF;
    constexpr int CPK = 4;                               // 16-byte chunks per row per 32-K step
    constexpr int PASSES = BM / T::ROWS_PER_DMA / NW;    // DMAs per wave per operand K-tile
    constexpr int STAGE = BM * BK_;                      // elements of one operand stage (32 KiB)
    constexpr int PIECE = T::ROWS_PER_DMA * BK_;         // elements one DMA instruction fills (1 KiB)
    static_assert(BM == BN && PASSES == 8 && PIECE * 2 == 1024, "square tile, 1 KiB DMA pieces");
    static_assert(STAGE == 4 * PASSES * PIECE, "a stage is 32 pieces, 8 per wave");
    static_assert(PASSES <= 63, "vmcnt holds 6 bits");

    __shared__ __attribute__((aligned(1024))) E smem[(SA + SB) * STAGE];
    E *const a_ring = smem;
    E *const b_ring = smem + SA * STAGE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int P = (int)gridDim.x;
    const int total = tiles_m * tiles_n;
    const int mine = (total - (int)blockIdx.x + P - 1) / P;  // tiles of this workgroup (>= 1)
    const int KT = K / BK_;  // at least 2

    // Tile i of this workgroup.  The grid sizes go through an opaque copy so
    // that the divisions of the tile order are done here, once per tile,
    // instead of keeping their reciprocals in vector registers across the K
    // loop.
    auto my_tile = [&](int i, int &tm, int &tn) {
        int gm = tiles_m, gn = tiles_n;
        asm volatile("" : "+s"(gm), "+s"(gn));
        tile_of_grouped<GM>((int)blockIdx.x + i * P, gm, gn, tm, tn);
    };
    // DMA sources: lane l of a wave fills physical chunk l mod 8 of row l / 8
    // of its pieces; successive pieces of a wave are 32 rows apart (a whole
    // number of swizzle periods), so its logical chunk kc is the same in all.
    static_assert((NW * T::ROWS_PER_DMA) % 16 == 0, "swizzle repeats per pass");
    uint32_t a_off[PASSES], b_off[PASSES];
    const char *a_src = nullptr, *b_src = nullptr;  // tile origins of the DMA stream's tile
    // Point the DMA stream at tile i of this workgroup: rows past M (N) are
    // clamped to the last row (they feed only D rows that are never stored).
    // The lane terms are recomputed here from an opaque lane index, so the
    // compiler cannot hoist them out of the tile loop into registers that
    // would have to live across the K loop.
    auto set_dma_tile = [&](int i) {
        int l = lane_id();
        asm volatile("" : "+v"(l));
        const int dr = l / T::RC;
        const int kc = (l % T::RC) ^ T::swz(T::ROWS_PER_DMA * wave + dr);
        int tm, tn;
        my_tile(i, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        a_src = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
        b_src = reinterpret_cast<const char *>(B + (int64_t)n0 * ldb);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
            a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda * 2 + 16 * kc);
            b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb * 2 + 16 * kc);
        }
    };
    // DMA stream: the refills run two K-tiles ahead of the matrix cores,
    // into the next tile during the last two K-tiles of a tile.  dsa, dsb:
    // the stages the next refills land in.
    int dsa = 0, dsb = 0;
    set_dma_tile(0);
    // descriptor of K-tile dk of the DMA stream's tile (live: the tile
    // exists; otherwise an empty range: every lane reads zero, no access)
    auto dma_rsrc = [&](const char *src, int dk, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(src + 2 * (int64_t)dk * BK_), (short)0,
                                                 live ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
    };
    auto next_dma_stage = [&]() {
        dsa = dsa + 1 == SA ? 0 : dsa + 1;
        dsb = dsb + 1 == SB ? 0 : dsb + 1;
    };
    auto dma_a = [&](__amdgpu_buffer_rsrc_t r, int p) {
        dma16<CPOL_CACHED>(r, a_ring + dsa * STAGE + (p * NW + wave) * PIECE, a_off[p]);
    };
    auto dma_b = [&](__amdgpu_buffer_rsrc_t r, int p) {
        dma16<CPOL_CACHED>(r, b_ring + dsb * STAGE + (p * NW + wave) * PIECE, b_off[p]);
    };

    const int frag_row = frag16_row_of(lane), frag_hi = frag16_hi_of(lane);
    V8 fa[2][TM], fb[2][TN];
    static_assert(T::swz(16) == T::swz(0) && WTM % 16 == 0 && WTN % 16 == 0, "swizzle period");
    int a_lane[2], b_lane[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        a_lane[kk] = T::off(wm * WTM + frag_row, kk * CPK + frag_hi);
        b_lane[kk] = T::off(wn * WTN + frag_row, kk * CPK + frag_hi);
    }
    auto read_frag = [&](int sa, int sb, int kk, int q, V8 *a, V8 *b) {
        if (q < TM)
            a[q] = *reinterpret_cast<const V8 *>(a_ring + sa * STAGE + a_lane[kk] + q * MF * BK_);
        else
            b[q - TM] = *reinterpret_cast<const V8 *>(b_ring + sb * STAGE + b_lane[kk] + (q - TM) * MF * BK_);
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int NFRAG = TM + TN;
    constexpr int SLOTS = TM * TN;
    auto frag_of_slot = [](int i) { return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN; };
    // One K-step: MFMA per slot; the next step's fragment read i after MFMA
    // RS·i; DMA pass (i-1)/8 of `which` (0: none, 1: A, 2: B) after every
    // eighth odd slot.
    auto step = [&](const V8 *a, const V8 *b, bool with_reads, int rsa, int rsb, int rkk, V8 *na, V8 *nb,
                    int which, __amdgpu_buffer_rsrc_t r, auto rs_tag) {
        constexpr int RS = decltype(rs_tag)::value;
        static_assert(SLOTS / RS >= NFRAG && SLOTS % 8 == 0, "reads and DMAs fit the slots");
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int ti = i / TN, tj = i % TN;
            acc[ti][tj] = Elem<E>::mfma(b[tj], a[ti], acc[ti][tj]);
            MFMA_FIRST();
            if (with_reads && i % RS == 0 && i / RS < NFRAG)
                read_frag(rsa, rsb, rkk, frag_of_slot(i / RS), na, nb);
            if (which && i % 8 == 1) {
                if (which == 1)
                    dma_a(r, i / 8);
                else
                    dma_b(r, i / 8);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using rs0_t = std::integral_constant<int, RS0>;
    using rs4_t = std::integral_constant<int, 4>;
    constexpr int X3 = SA == 3 ? 1 : 2;  // operand with three stages: refilled in K-step 0
    constexpr int Y2 = 3 - X3;           // the other: refilled in K-step 1

    // Staged epilogue of tile `ti` in the three-stage operand's stage sa
    // (A) or sb (B).
    static_assert(TM % 4 == 0 && WTM / 4 * WTN == 8 * PIECE, "a quarter of a wave block fills its eight pieces");
    auto epilogue = [&](int ti, int sa, int sb) __attribute__((always_inline)) {
        int tm, tn;
        my_tile(ti, tm, tn);
        const int row0 = tm * BM + wm * WTM, col0 = tn * BN + wn * WTN;
        // this wave's pieces, 4·PIECE apart; piece q (0..7) of a quarter holds
        // its rows 4q..4q+3, 256 bytes each
        E *const st = (X3 == 1 ? a_ring + sa * STAGE : b_ring + sb * STAGE) + wave * PIECE;
        auto piece = [&](int q) { return st + q * 4 * PIECE; };
        int l = lane_id();
        asm volatile("" : "+v"(l));  // opaque: the lane terms below are not hoisted out of the tile loop
        const int fr = l & 15, fh = l >> 4;     // accumulator lane: D row fr, columns 4·fh..4·fh+3
        const int rr = l >> 4, rc = l & 15;     // store lane: row rr of a piece, 16-byte chunk rc
        const bool inside = dvec && row0 + WTM <= M && col0 + WTN <= N;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int i = 0; i < TM / 4; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const f32x4 v = acc[2 * h + i][j];
                    acc[2 * h + i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    V4 e;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[r] = (E)v[r];  // round to nearest even
                    const int c = j * MF + 4 * fh;  // column in the wave block
                    E *dst = piece(4 * i + (fr >> 2)) + (fr & 3) * (WTN) + (((c >> 3) ^ fr) << 3) + (c & 7);
                    *reinterpret_cast<V4 *>(dst) = e;
                }
            // Every DMA of this wave has landed before its first store:
            // the vector-memory counter also counts stores, so the next
            // tile's first wait, which only needs those DMAs, is dropped
            // instead of draining this epilogue's stores.
            if (h == 0)
                wait_vmem<0>();
            const int rbase = row0 + 32 * h;
            const int col = col0 + 8 * rc;
            if (inside) {
                E *dst = D + (int64_t)(rbase + rr) * ldd + col;
                V8 v[8];  // all eight LDS reads ahead of the stores
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    v[q] = *reinterpret_cast<const V8 *>(piece(q) + rr * WTN + ((rc ^ ((4 * q + rr) & 15)) << 3));
                if (dvec == D_VEC_NT) {
                    const auto r = d_block_rsrc(D + (int64_t)row0 * ldd + col0);
                    const uint32_t voff = (uint32_t)(rr * ldd * 2 + 16 * rc);
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        store16_nt(v[q], r, voff, (uint32_t)((32 * h + 4 * q) * ldd * 2));
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        *reinterpret_cast<V8 *>(dst + (int64_t)(4 * q) * ldd) = v[q];
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const V8 v = *reinterpret_cast<const V8 *>(piece(q) + rr * WTN + ((rc ^ ((4 * q + rr) & 15)) << 3));
                    const int row = rbase + 4 * q + rr;
                    if (row < M) {
                        E *dst = D + (int64_t)row * ldd + col;
                        if (dvec && col + 7 < N) {
                            *reinterpret_cast<V8 *>(dst) = v;
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (col + e < N)
                                    dst[e] = v[e];
                        }
                    }
                }
            }
        }
    };

    // prologue: K-tiles 0 and 1 of the first tile; wait for K-tile 0
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const auto ra = dma_rsrc(a_src, e, true), rb = dma_rsrc(b_src, e, true);
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            dma_a(ra, p);
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            dma_b(rb, p);
        next_dma_stage();
    }
    wait_vmem<2 * PASSES>();
    barrier_lds();
#pragma unroll
    for (int q = 0; q < NFRAG; ++q)
        read_frag(0, 0, 0, q, fa[0], fb[0]);

    int sa = 0, sb = 0;  // stages of the K-tile being multiplied
    // One K-tile: K-step 0 with the three-stage operand's refill (K-tile dk
    // of the DMA stream's tile), the wait for the next K-tile and the
    // barrier that drains this one's stages, K-step 1 with the other
    // operand's refill, reading K-step 0 of the next K-tile (unless `last`).
    bool fresh = false;  // the first K-tile after an epilogue, whose next K-tile landed before the stores
    auto k_tile = [&](int dk, bool live, bool last) __attribute__((always_inline)) {
        step(fa[0], fb[0], true, sa, sb, 1, fa[1], fb[1], X3, dma_rsrc(X3 == 1 ? a_src : b_src, dk, live),
             rs0_t{});
        if (!fresh)
            wait_vmem<PASSES>();  // all but that refill: the next K-tile has landed (this wave's part)
        fresh = false;
        barrier_lds();        // ... for every wave; this K-tile's stages are drained
        const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb + 1 == SB ? 0 : sb + 1;
        step(fa[1], fb[1], !last, sa1, sb1, 0, fa[0], fb[0], Y2, dma_rsrc(Y2 == 1 ? a_src : b_src, dk, live),
             rs4_t{});
        next_dma_stage();
        sa = sa1;
        sb = sb1;
    };
    for (int ci = 0; ci < mine; ++ci) {
        for (int kt = 0; kt + 2 < KT; ++kt)
            k_tile(kt + 2, true, false);
        // the last two K-tiles refill K-tiles 0 and 1 of the next tile
        const bool more = ci + 1 < mine;
        if (more)
            set_dma_tile(ci + 1);
        k_tile(0, more, false);
        const int esa = sa, esb = sb;  // stages of the last K-tile: the staging memory
        k_tile(1, more, !more);
        epilogue(ci, esa, esb);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging reads are done
        fresh = true;
    }
    wait_vmem<0>();  // no DMA or store may be outstanding when the wave ends
    if constexpr (STAMP) {
        barrier_lds();  // every wave is done
        const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0)
            stamps[3 * blockIdx.x + 1] = t1;
    }
}

// ------------------------------------------------------------------------
// Block-scaled FP8 GEMM ("TIRx Layout API", section "Scale Factor 布局": a
// block-scaled MMA reads, besides its operands, one 8-bit scale factor per
// group of K elements of every row, and the scale factors are laid out so
// that each lane window that consumes a row sees its row's factors).  Read as
// OCP MX: E4M3 operand bytes, one UE8M0 scale byte per 32 K elements of a
// row, fp32 accumulation, fp16 output rounded to nearest even.
//
// gfx950 does the scaling inside the matrix core: v_mfma_scale_f32_32x32x64
// takes per lane a 32-byte operand slice and a 32-bit scale register whose
// low byte scales one 32-element block.  Its lane map (probed on the device):
// lane l = r + 32·h holds row r; its bytes 0..15 are K 16h..16h+15 and bytes
// 16..31 are K 32+16h..32+16h+15 of the instruction's 64 K, so it reads
// 16-byte chunks h and 2+h of the K-step; and the scale byte of lane r + 32·h
// applies to block h (K 32h..32h+31) of row r, on either operand.  With the
// MFMA inputs swapped as in the fp16 kernels (B feeds the first input), the
// accumulator map is the 32×32 one of v_mfma_f32_32x32x16_f16.
//
// Everything else follows gemm_dma3_kernel: a 256×256 tile, four waves of
// 128×128, 128-byte operand rows in LDS (128 K per stage, two 64-K MFMA
// K-steps per stage) with the same swizzle and source-side DMA addressing,
// three A stages and two B stages.  Per iteration t:
//   K-step 0: A(t+2) is DMAed while both halves of K-step 1's fragments
//             are read (in the step's first half);
//   wait until all but A(t+2) has landed; barrier; (at the first K-tile of
//   a group, and the second in groups of four) the scale words of the next
//   group are loaded;
//   K-step 1: B(t+2) is DMAed while the fragments of K-tile t+1's K-step 0
//             are read.
// A scale word holds the four blocks of one row in one K-tile; lane r + 32·h
// feeds the MFMA of K-step kk the byte for block 2·kk + h, and blocks at or
// past K/32 (the tail of the last K-tile, whose operand bytes are zero) read
// as 2^0 instead of whatever the padding holds.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element encodings (OCP MX defines two for FP8): FMT = a + 2·b with a, b the
// encodings of A and B, 0 for E4M3 and 1 for E5M2 (the instruction's format
// codes for fp8 and bf8).  The scaled MFMA takes the format of its first
// source (here B, as the MFMA inputs are swapped) and of its second (A).
#define MX_FMT_A(F) ((F) & 1)
#define MX_FMT_B(F) ((F) >> 1)

__host__ __device__ constexpr int mx_row_of(int l) { return l & 31; }
__host__ __device__ constexpr int mx_chunk_of(int l, int kk, int half) { return 4 * kk + 2 * half + (l >> 5); }
constexpr bool mx_fragment_covers_k_step()
{
    // every (row, K) of a 32-row, 64-K step is read by exactly one lane byte
    bool seen[32 * 64] = {};
    for (int l = 0; l < 64; ++l)
        for (int half = 0; half < 2; ++half)
            for (int e = 0; e < 16; ++e) {
                const int k = 16 * mx_chunk_of(l, 0, half) + e;
                const int idx = mx_row_of(l) * 64 + k;
                if (k >= 64 || seen[idx])
                    return false;
                seen[idx] = true;
            }
    return true;
}
static_assert(mx_fragment_covers_k_step(), "scaled-MFMA fragment reads must cover the K-step once");

// Scale words of G consecutive K-tiles, loaded by one buffer load.
template <int G>
struct MxGroup;
template <>
struct MxGroup<2> {
    typedef unsigned type __attribute__((ext_vector_type(2)));
    __device__ static type load(__amdgpu_buffer_rsrc_t r, int off)
    {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
};
template <>
struct MxGroup<4> {
    typedef unsigned type __attribute__((ext_vector_type(4)));
    __device__ static type load(__amdgpu_buffer_rsrc_t r, int off)
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
};

// Where a scale word lives.  Row-major (PK false): row r's byte of block b
// at r·lds + b, so the word of K-tile t (blocks 4t .. 4t+3) at r·lds + 4t.
// Packed (PK true): 512-byte chunks of 32 rows × 16 blocks, chunk (r/32,
// b/16) at (r/32)·lds + (b/16)·512 (lds = the bytes of one 32-row group:
// 512 per 16 blocks of K), row r%32 at 16·(r%32) inside it — the
// 32-row × scale-block atom the matrix core consumes, so that the words of
// a 32-row fragment for four K-tiles are 512 contiguous bytes instead of 32
// cache lines.  Offsets are relative to the tile's first row (a multiple of
// 32).
template <bool PK>
__device__ inline uint32_t mx_row_off(int r, int64_t lds)
{
    return PK ? (uint32_t)((r >> 5) * lds + (r & 31) * 16) : (uint32_t)(r * lds);
}
template <bool PK>
__device__ inline uint32_t mx_ktile_off(int t)
{
    return PK ? (uint32_t)((t >> 2) * 512 + (t & 3) * 4) : (uint32_t)(4 * t);
}
// Buffer descriptor over the scale rows of rows [r0, rows) (r0 a multiple of
// 32): rows past `rows` read as zero words (row-major) or the packed pad.
template <bool PK>
__device__ inline __amdgpu_buffer_rsrc_t mx_scale_rsrc(const uint8_t *S, int r0, int rows, int64_t lds)
{
    const int64_t base = PK ? (int64_t)(r0 >> 5) * lds : (int64_t)r0 * lds;
    const int64_t bytes = PK ? (int64_t)((rows + 31) / 32 - (r0 >> 5)) * lds : (int64_t)(rows - r0) * lds;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(S + base), (short)0, (int)imin64(bytes, DMA_RANGE),
                                             BUFFER_RSRC_WORD3);
}

template <int BM, int BN, int WM, int WN, int MX_GROUP, bool PK, int FMT>
__global__ __launch_bounds__(WM *WN * 64) TG_WAVES_PER_SIMD(1) void gemm_mxf8_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ SB, _Float16 *__restrict__ D, int M, int N, int K, int64_t lda,
    int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd, int tiles_m, int tiles_n, int dvec)
{
    using E = _Float16;
    using V4 = Elem<E>::v4;
    constexpr int BKB = 128;  // K elements (= bytes) per stage row
    constexpr int SA_ = 3, SB_ = 2;
    using T = OperandTile<64>;  // 128-byte rows; T::off counts 2-byte units
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KSTEPS = BKB / 64;
    constexpr int A_PASSES = BM / T::ROWS_PER_DMA / NW, B_PASSES = BN / T::ROWS_PER_DMA / NW;
    constexpr int STAGE_A = BM * BKB, STAGE_B = BN * BKB;  // bytes
    constexpr int NFRAG = TM + TN;
    constexpr int SLOTS = TM * TN;
    static_assert(KSTEPS == 2 && SLOTS == 2 * NFRAG, "two K-steps; one fragment half read per slot");
    static_assert((BM / T::ROWS_PER_DMA) % NW == 0 && (BN / T::ROWS_PER_DMA) % NW == 0,
                  "DMA row groups must split evenly over the waves");
    static_assert(SA_ * STAGE_A + SB_ * STAGE_B <= 160 * 1024, "LDS budget");
    static_assert(2 * NFRAG + A_PASSES + B_PASSES + A_PASSES <= 63, "vmcnt holds 6 bits");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SA_ * STAGE_A + SB_ * STAGE_B];
    uint8_t *const a_ring = smem;
    uint8_t *const b_ring = smem + SA_ * STAGE_A;

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int dr = lane / T::RC, dpc = lane % T::RC;
    // Successive passes of a wave are NW·ROWS_PER_DMA = 32 rows apart, a
    // whole number of swizzle periods, so a lane fetches the same logical
    // chunk in every pass.
    static_assert((NW * T::ROWS_PER_DMA / T::ROWS_PER_LINE) % T::RC == 0, "swizzle repeats per pass");
    const int kc = dpc ^ T::swz(T::ROWS_PER_DMA * wave + dr);
    uint32_t a_off[A_PASSES], b_off[B_PASSES];
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda + 16 * kc);
    }
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb + 16 * kc);
    }
    const uint8_t *a_tile = A + (int64_t)m0 * lda;
    const uint8_t *b_tile = B + (int64_t)n0 * ldb;
    const int KT = (K + BKB - 1) / BKB;
    const int nblk = K / 32;

    struct Op {
        __amdgpu_buffer_rsrc_t r;
        uint8_t *dst;
        int klim;
    };
    auto op_a = [&](int t) {
        Op o;
        o.r = __builtin_amdgcn_make_buffer_rsrc((void *)(a_tile + t * BKB), (short)0, DMA_RANGE,
                                                BUFFER_RSRC_WORD3);
        o.dst = a_ring + (t % SA_) * STAGE_A;
        o.klim = t < KT ? K - t * BKB : 0;
        return o;
    };
    auto op_b = [&](int t) {
        Op o;
        o.r = __builtin_amdgcn_make_buffer_rsrc((void *)(b_tile + t * BKB), (short)0, DMA_RANGE,
                                                BUFFER_RSRC_WORD3);
        o.dst = b_ring + (t % SB_) * STAGE_B;
        o.klim = t < KT ? K - t * BKB : 0;
        return o;
    };
    auto dma_a = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BKB,
                           16 * kc < o.klim ? a_off[p] : DMA_OOB);
    };
    auto dma_b = [&](const Op &o, int p) {
        dma16<CPOL_CACHED>(o.r, o.dst + (p * NW + wave) * T::ROWS_PER_DMA * BKB,
                           16 * kc < o.klim ? b_off[p] : DMA_OOB);
    };

    // Scale words: a buffer over the rows from m0 (n0) on, so rows past M
    // (N), which feed only unstored outputs, read as zero words (or the
    // packed layout's pad).
    const int srow = mx_row_of(lane), shalf = lane >> 5;
    const __amdgpu_buffer_rsrc_t sa_rsrc = mx_scale_rsrc<PK>(SA, m0, M, ldsa);
    const __amdgpu_buffer_rsrc_t sb_rsrc = mx_scale_rsrc<PK>(SB, n0, N, ldsb);
    uint32_t sw_a[1][TM] = {}, sw_b[1][TN] = {};  // scale words of the current K-tile
    // Grouped scale words: one MX_GROUP·4-byte load per lane per fragment
    // pair covers MX_GROUP K-tiles — lanes 0..31 take row r of the pair's
    // first fragment, lanes 32..63 row r of its second — so each load
    // touches one cache line per row for MX_GROUP K-tiles instead of one
    // per K-tile (scattered 4-byte loads cost the address unit per line);
    // a swap of the two lane halves (v_permlane32_swap) then hands every
    // lane its own fragment's word.
    constexpr int NPA = TM / 2, NPB = TN / 2;
    const uint32_t sa_poff = mx_row_off<PK>(wm * WTM + (lane >> 5) * 32 + srow, ldsa);
    const uint32_t sb_poff = mx_row_off<PK>(wn * WTN + (lane >> 5) * 32 + srow, ldsb);
    const uint32_t sa_pair = mx_row_off<PK>(64, ldsa), sb_pair = mx_row_off<PK>(64, ldsb);  // 64 rows on
    using GroupWord = typename MxGroup<MX_GROUP>::type;
    GroupWord gw[2][NPA + NPB] = {};  // [current, next group][pair]
    // Pairs [lo, hi) of the group starting at K-tile t0 (A pairs first).
    auto load_group = [&](int t0, GroupWord *g, int lo, int hi) {
#pragma unroll
        for (int p = 0; p < NPA; ++p)
            if (p >= lo && p < hi)
                g[p] = MxGroup<MX_GROUP>::load(sa_rsrc, (int)(sa_poff + p * sa_pair + mx_ktile_off<PK>(t0)));
#pragma unroll
        for (int p = 0; p < NPB; ++p)
            if (NPA + p >= lo && NPA + p < hi)
                g[NPA + p] = MxGroup<MX_GROUP>::load(sb_rsrc, (int)(sb_poff + p * sb_pair + mx_ktile_off<PK>(t0)));
    };
    // Words of K-tile t (index j of group g) into sw_a[0] / sw_b[0], ready
    // for the MFMA: blocks at or past K/32 (the tail of a partial last
    // K-tile, and K-tiles past the end) become 2^0 by a wave-uniform byte
    // mask, and each lane shifts its word right by 8·h, so that byte 2·kk
    // (the MFMA's byte select for K-step kk) holds block 4t + 2kk + h.
    auto unpack_group = [&](const GroupWord *g, int j, int t) {
        const int nv = nblk - 4 * t;
        const uint32_t keep = nv >= 4 ? 0xffffffffu : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
        const uint32_t unit = 0x7f7f7f7fu & ~keep;
        const uint32_t sh = 8 * shalf;
#pragma unroll
        for (int p = 0; p < NPA + NPB; ++p) {
            const uint32_t v = ((uint32_t)g[p][j] & keep) | unit;
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            uint32_t *dst = p < NPA ? &sw_a[0][2 * p] : &sw_b[0][2 * (p - NPA)];
            dst[0] = r[0] >> sh;
            dst[1] = r[1] >> sh;
        }
    };

    i32x8 fa[2][TM], fb[2][TN];
    // per-lane byte offsets of chunk (kk, half) in a stage; the swizzle
    // repeats every 16 rows, so fragment q sits a constant q·32 rows further
    static_assert(T::swz(16) == T::swz(0) && WTM % 16 == 0 && WTN % 16 == 0, "swizzle period");
    int a_lane[KSTEPS][2], b_lane[KSTEPS][2];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            a_lane[kk][half] = 2 * T::off(wm * WTM + srow, mx_chunk_of(lane, kk, half));
            b_lane[kk][half] = 2 * T::off(wn * WTN + srow, mx_chunk_of(lane, kk, half));
        }
    auto read_frag = [&](int sa, int sb, int kk, int q, int half, i32x8 *a, i32x8 *b) {
        const uint8_t *src = q < TM ? a_ring + sa * STAGE_A + a_lane[kk][half] + q * 32 * BKB
                                    : b_ring + sb * STAGE_B + b_lane[kk][half] + (q - TM) * 32 * BKB;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(src);
        i32x8 &f = q < TM ? a[q] : b[q - TM];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * half + e] = v[e];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    auto frag_of_slot = [](int i) { return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN; };
    // One K-step of K-tile t: MFMA per slot; DMA passes [0, n) of `o` in the
    // odd slots.  The next step's fragments: in K-step 0 (whose reads must
    // land before the barrier that follows it) both halves of fragment i
    // after each of the first NFRAG MFMAs, so the last read has half a step
    // to land; in K-step 1 (read by the next K-tile's first MFMAs) half i%2
    // of fragment i/2 after MFMA i.
    auto step = [&](const i32x8 *a, const i32x8 *b, const uint32_t *wa, const uint32_t *wb, int t, int kk,
                    bool with_reads, int rsa, int rsb, int rkk, i32x8 *na, i32x8 *nb, const Op *o, bool is_a,
                    int n) {
        (void)t;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int ti = i / TN, tj = i % TN;
            // the scale byte of K-step kk is byte 2·kk of the prepared word
            if (kk == 0)
                acc[ti][tj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b[tj], a[ti], acc[ti][tj], MX_FMT_B(FMT), MX_FMT_A(FMT), 0, (int)wb[tj], 0, (int)wa[ti]);
            else
                acc[ti][tj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b[tj], a[ti], acc[ti][tj], MX_FMT_B(FMT), MX_FMT_A(FMT), 2, (int)wb[tj], 2, (int)wa[ti]);
            MFMA_FIRST();
            if (with_reads && kk == 0) {
                if (i < NFRAG) {
                    read_frag(rsa, rsb, rkk, frag_of_slot(i), 0, na, nb);
                    read_frag(rsa, rsb, rkk, frag_of_slot(i), 1, na, nb);
                }
            } else if (with_reads) {
                read_frag(rsa, rsb, rkk, frag_of_slot(i / 2), i % 2, na, nb);
            }
            if (o && (i % 2) == 1 && i / 2 < n) {
                if (is_a)
                    dma_a(*o, i / 2);
                else
                    dma_b(*o, i / 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The K loop runs over KTP = KT rounded up to a multiple of MX_GROUP (at
    // least one group) in groups of K-tiles; a K-tile past KT reads zero
    // operands and gets unit scales (its blocks lie past K/32), so it adds
    // nothing.  Scale-word group i holds K-tiles G·i .. G·i+G-1.  Where KT is
    // not a multiple of G the last group's words past the last K-tile lie
    // past the end of a scale row: they read the next row's bytes or, past
    // the buffer, zero — the buffer unit checks each dword of a multi-dword
    // load on its own (probed), so the group's words in range are intact.
    static_assert(MX_GROUP == 2 || MX_GROUP == 4, "groups of two or four K-tiles");
    const int KTP = KT < MX_GROUP ? MX_GROUP : (KT + MX_GROUP - 1) / MX_GROUP * MX_GROUP;
    load_group(0, gw[0], 0, NPA + NPB);
    // prologue DMAs: A(0), B(0), A(1), B(1)
    {
        const Op a0 = op_a(0), b0 = op_b(0), a1 = op_a(1), b1 = op_b(1);
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p)
            dma_a(a0, p);
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p)
            dma_b(b0, p);
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p)
            dma_a(a1, p);
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p)
            dma_b(b1, p);
    }
    wait_vmem<A_PASSES + B_PASSES>();
    barrier_lds();
    unpack_group(gw[0], 0, 0);
#pragma unroll
    for (int q = 0; q < NFRAG; ++q) {
        read_frag(0, 0, 0, q, 0, fa[0], fb[0]);
        read_frag(0, 0, 0, q, 1, fa[0], fb[0]);
    }

    int sa = 0, sb = 0;
    // K-tile t (t < KT-1): K-step 0 with A(t+2); wait and barrier; `extra`
    // (the next group's loads, which then have until the following K-tile's
    // wait to land); K-step 1 with B(t+2) and the first fragments of t+1;
    // `after` (unpack the scale words of t+1).
    auto k_tile = [&](int t, auto extra, auto after) __attribute__((always_inline)) {
        const Op an = op_a(t + 2);
        step(fa[0], fb[0], sw_a[0], sw_b[0], t, 0, true, sa, sb, 1, fa[1], fb[1], &an, true, A_PASSES);
        wait_vmem<A_PASSES>();  // B(t+1), A(t+1) and the scale loads before them have landed
        barrier_lds();
        extra();
        const Op b2 = op_b(t + 2);
        const int sa1 = sa + 1 == SA_ ? 0 : sa + 1, sb1 = sb + 1 == SB_ ? 0 : sb + 1;
        step(fa[1], fb[1], sw_a[0], sw_b[0], t, 1, true, sa1, sb1, 0, fa[0], fb[0], &b2, false, B_PASSES);
        sa = sa1;
        sb = sb1;
        after();
    };
    auto nothing = [] {};
    // Group (kt .. kt+G-1): its first K-tiles load the next group (the last
    // group reloads one in range; its words go unused) — in groups of four,
    // the A pairs in the first K-tile and the B pairs in the second, so that
    // fewer scattered loads stand in front of one K-tile's DMAs.  The last
    // K-tile runs like the others: its trailing DMAs are past K (no memory
    // access) and its trailing fragment reads are never used.
    constexpr int SPREAD = MX_GROUP == 4 ? 2 : 1;  // K-tiles the next group's loads spread over
    constexpr int PER = (NPA + NPB) / SPREAD;
    static_assert((NPA + NPB) % SPREAD == 0 && SPREAD < MX_GROUP, "the loads end before the group's last K-tile");
    for (int kt = 0; kt < KTP; kt += MX_GROUP) {
        const int tnext = imax(0, imin(kt + MX_GROUP, KT - 1));
        k_tile(kt, [&] { load_group(tnext, gw[1], 0, PER); }, [&] { unpack_group(gw[0], 1, kt + 1); });
#pragma unroll
        for (int j = 1; j + 1 < MX_GROUP; ++j)
            k_tile(kt + j, [&] { if (j < SPREAD) load_group(tnext, gw[1], j * PER, (j + 1) * PER); },
                   [&] { unpack_group(gw[0], j + 1, kt + j + 1); });
        k_tile(kt + MX_GROUP - 1, nothing, [&] {
#pragma unroll
            for (int p = 0; p < NPA + NPB; ++p)
                gw[0][p] = gw[1][p];
            unpack_group(gw[0], 0, kt + MX_GROUP);
        });
    }
    wait_vmem<0>();

    // staged epilogue, as in gemm_dma3_kernel
    static_assert(NW * WTM * WTN * 2 <= SA_ * STAGE_A + SB_ * STAGE_B, "staging fits in the stage memory");
    constexpr int SROW = WTN;
    constexpr int SCH = WTN / 8;
    static_assert((SCH & (SCH - 1)) == 0 && SCH >= 2, "chunk swizzle needs a power of two");
    auto stage_off = [](int r, int chunk) { return r * SROW + ((chunk ^ (r & (SCH - 1))) << 3); };
    barrier_lds();
    E *stg = reinterpret_cast<E *>(smem) + wave * WTM * WTN;
    const int elane = lane_id();
    const int frag_row = frag_row_of(elane), frag_hi = frag_hi_of(elane);
    static_assert(TM == 4, "one 32-row fragment row per quarter");
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                V4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (E)acc[i][j][g * 4 + r];  // round to nearest even
                const int r = i * 32 + frag_row;
                const int c = j * 32 + g * 8 + frag_hi * 4;
                *reinterpret_cast<V4 *>(stg + stage_off(r, c / 8) + (c & 7)) = h;
            }
        store_staged_block<E, WTM, WTN, decltype(stage_off), 32>(stg, stage_off, D, ldd, m0 + wm * WTM,
                                                                 n0 + wn * WTN, M, N, dvec, elane, 32 * i);
    }
}

// 64×128 tiles of the block-scaled GEMM, for small M (M <= 64: one 64-row
// tile row covers all of M, so each workgroup streams its own 128-row band
// of B exactly once — the fp16 strip tiles' argument: the shape is bound by
// reading B from HBM, not by the matrix cores) and for problems with too
// few 256×256 tiles to occupy the GPU (tiles_m × tiles_n workgroups, column
// strips innermost).  Four waves
// split the band by columns (64×32 each: two 32-row A fragments, one B
// fragment per 64-K step); STAGES LDS stages hold, per 128-K tile, A's 64
// and B's 128 operand rows (same swizzle and source-side DMA addressing as
// the 256×256 kernel).  The scale words ride the same DMA stream, four
// K-tiles at a time: at the first K-tile of a group of four, one
// 16-byte-per-lane DMA per wave (wave 0: A rows 0..63, waves 1 and 2: B
// rows 0..63 and 64..127) fills one of three scale slots (scattered scale
// loads cost the address unit per cache line: a DMA per K-tile cost 18% of
// the time); at the other K-tiles, and always in wave 3, an empty DMA into
// a spare slot keeps every wave's count of DMAs in flight the same; each
// lane copies its fragment rows' four words into registers at the group's
// first K-tile and picks the K-tile's word from them after that.  B's
// DMAs stream past the caches; the workgroups on XCD x start their K loop at
// K-tile x·KT/8 (rounded down to a group) and wrap around, so the eight XCDs
// read different column bands of B's rows at a time.  Each K-tile: wait for
// its DMAs, barrier, refill the stage drained by the barrier with K-tile
// t+STAGES-1 (K-tiles past the end get empty ranges: no memory access), then
// the scale words (masked to 2^0 past K/32, shifted for the lane half) and
// two 64-K steps of two MFMAs.
template <int STAGES, bool PK, int FMT>
__global__ __launch_bounds__(256) void gemm_mxf8_strip_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ SB, _Float16 *__restrict__ D, int M, int N, int K, int64_t lda,
    int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd, int tiles_n, int dvec)
{
    using E = _Float16;
    using V4 = Elem<E>::v4;
    constexpr int BM = 64, BN = 128, NW = 4, BKB = 128;
    constexpr int WTM = BM, WTN = BN / NW;       // 64×32 per wave
    constexpr int TM = WTM / 32, TN = WTN / 32;  // 2 A fragments, 1 B fragment
    using T = OperandTile<64>;                   // 128-byte rows; T::off counts 2-byte units
    constexpr int A_PASSES = BM / T::ROWS_PER_DMA / NW, B_PASSES = BN / T::ROWS_PER_DMA / NW;
    constexpr int DPT = A_PASSES + B_PASSES + 1;  // DMAs per K-tile per wave (the last: scale words)
    constexpr int STAGE_A = BM * BKB, STAGE_B = BN * BKB;  // bytes
    constexpr int STAGE = STAGE_A + STAGE_B;
    constexpr int SC_SLOT = 16 * 64 * NW;  // scale words of 4 K-tiles: 16 bytes per lane and wave
    static_assert(STAGES >= 2 && STAGES <= 5, "a scale slot is rewritten 3 groups later");
    static_assert(STAGES * STAGE + 4 * SC_SLOT <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 1) * DPT <= 63, "vmcnt holds 6 bits");
    static_assert(NW * WTM * WTN * 2 <= STAGES * STAGE, "staging fits in the stage memory");
    static_assert((BM / T::ROWS_PER_DMA) % NW == 0 && (BN / T::ROWS_PER_DMA) % NW == 0,
                  "DMA row groups must split evenly over the waves");
    static_assert(T::swz(16) == T::swz(0) && WTN % 16 == 0, "swizzle period");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + 4 * SC_SLOT];
    uint8_t *const sc_ring = smem + STAGES * STAGE;  // three slots, then one that empty DMAs fill

    // tile (tm, tn) of a tiles_m × tiles_n grid of 64×128 tiles, column
    // strips innermost
    const int tm = (int)(blockIdx.x / (unsigned)tiles_n), tn = (int)(blockIdx.x % (unsigned)tiles_n);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int dr = lane / T::RC, dpc = lane % T::RC;
    uint32_t a_off[A_PASSES], b_off[B_PASSES];
    int a_kc[A_PASSES], b_kc[B_PASSES];
#pragma unroll
    for (int p = 0; p < A_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        a_kc[p] = dpc ^ T::swz(t);
        a_off[p] = (uint32_t)(imin(t, M - 1 - m0) * lda + 16 * a_kc[p]);
    }
#pragma unroll
    for (int p = 0; p < B_PASSES; ++p) {
        const int t = T::ROWS_PER_DMA * (p * NW + wave) + dr;
        b_kc[p] = dpc ^ T::swz(t);
        b_off[p] = (uint32_t)(imin(t, N - 1 - n0) * ldb + 16 * b_kc[p]);
    }
    const uint8_t *a_band = A + (int64_t)m0 * lda;
    const uint8_t *b_band = B + (int64_t)n0 * ldb;
    // scale rows from row m0 of A and row n0 of B; rows past M (N) read zero
    // words or the packed layout's pad (they feed only unstored outputs)
    const __amdgpu_buffer_rsrc_t sc_rsrc =
        wave == 0 ? mx_scale_rsrc<PK>(SA, m0, M, ldsa) : mx_scale_rsrc<PK>(SB, n0, N, ldsb);
    const uint32_t sc_off = wave == 0 ? mx_row_off<PK>(lane, ldsa) : mx_row_off<PK>((wave - 1) * 64 + lane, ldsb);

    const int KT = (K + BKB - 1) / BKB;
    const int nblk = K / 32;
    // a multiple of 4, so that the K-tiles of each group of four are visited
    // together (the group holding the last K-tile may be shorter)
    const int kstart = KT > 0 ? ((int)(blockIdx.x % 8) * KT / 8) & ~3 : 0;
    // K-tile index of loop step t (steps past KT are empty)
    auto ktile = [&](int t) { return t < KT ? (t + kstart) % KT : t; };
    // scale slot of loop step t: groups in visiting order, modulo 3 (a slot
    // is refilled STAGES-1 <= 4 steps before its group's first step, by
    // which time the group three back has been read: at most one group, the
    // one that ends at the last K-tile, is shorter than four)
    const int before_wrap = KT - kstart;
    auto slot = [&](int t) {
        const int g = t < before_wrap ? t / 4 : (before_wrap + 3) / 4 + (t - before_wrap) / 4;
        return g % 3;
    };
    auto issue = [&](int t) {
        const int kt = ktile(t);
        const bool live = t < KT;
        uint8_t *st = smem + (t % STAGES) * STAGE;
        const int klim = live ? K - kt * BKB : 0;  // valid bytes of each row in this K-tile
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a_band + (int64_t)kt * BKB), (short)0, live ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(b_band + (int64_t)kt * BKB), (short)0, live ? DMA_RANGE : 0, BUFFER_RSRC_WORD3);
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p)
            dma16<CPOL_CACHED>(ra, st + (p * NW + wave) * T::ROWS_PER_DMA * BKB,
                               16 * a_kc[p] < klim ? a_off[p] : DMA_OOB);
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p)
            dma16<CPOL_STREAM>(rb, st + STAGE_A + (p * NW + wave) * T::ROWS_PER_DMA * BKB,
                               16 * b_kc[p] < klim ? b_off[p] : DMA_OOB);
        // at a group's first K-tile, 16 bytes per row: its four words (words
        // past the row's last K-tile are never used); otherwise an empty DMA
        // into the spare slot keeps the count
        const bool first = live && wave < 3 && kt % 4 == 0;
        dma16<CPOL_CACHED>(sc_rsrc, sc_ring + (first ? slot(t) : 3) * SC_SLOT + wave * 1024,
                           first ? sc_off + mx_ktile_off<PK>(kt) : DMA_OOB);
    };

    const int srow = mx_row_of(lane), shalf = lane >> 5;
    int a_lane[2][2], b_lane[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            a_lane[kk][half] = 2 * T::off(srow, mx_chunk_of(lane, kk, half));
            b_lane[kk][half] = STAGE_A + 2 * T::off(wave * WTN + srow, mx_chunk_of(lane, kk, half));
        }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    // the scale words of the current group of four K-tiles: the four words of
    // each of the lane's fragment rows (row r's words sit at bytes 16·r ..
    // 16·r+15 of the slot, B's rows after A's 64), read from LDS once, at the
    // group's first K-tile — each lane reads its row's whole 16 bytes, so
    // sixteen consecutive rows fill all 64 banks once — and kept in
    // registers for the group's other K-tiles, whose scale selection then
    // waits on no LDS read
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 ga[TM], gb[TN];

#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
        issue(t);
    for (int t = 0; t < KT; ++t) {
        wait_vmem<(STAGES - 2) * DPT>();  // this wave's DMAs of K-tile t have landed
        barrier_lds();                    // ... every wave's; the stage of t-1 is drained
        issue(t + STAGES - 1);
        const uint8_t *st = smem + (t % STAGES) * STAGE;
        // a group starts at every K-tile that is a multiple of four (the loop
        // starts at one and wraps around to K-tile 0); its words landed with
        // this K-tile's DMAs
        const int kt = ktile(t);
        if (kt % 4 == 0) {
            const u32x4 *sw = reinterpret_cast<const u32x4 *>(sc_ring + slot(t) * SC_SLOT);
#pragma unroll
            for (int q = 0; q < TM; ++q)
                ga[q] = sw[q * 32 + srow];
#pragma unroll
            for (int q = 0; q < TN; ++q)
                gb[q] = sw[64 + wave * WTN + q * 32 + srow];
        }
        // scale words: blocks at or past K/32 become 2^0 (the operand bytes
        // there are zero, the padding's scale bytes may be anything); lane
        // r + 32·h shifts by 8·h so that byte 2·kk holds block 4·kt + 2·kk + h;
        // word kt mod 4 of the group's four is a wave-uniform choice
        const int nv = nblk - 4 * kt;
        const uint32_t keep = nv >= 4 ? 0xffffffffu : (1u << (8 * nv)) - 1u;
        const uint32_t unit = 0x7f7f7f7fu & ~keep;
        const int wsel = kt % 4;
        auto pick = [wsel](const u32x4 &v) {
            return wsel == 0 ? v[0] : wsel == 1 ? v[1] : wsel == 2 ? v[2] : v[3];
        };
        uint32_t wa[TM], wb[TN];
#pragma unroll
        for (int q = 0; q < TM; ++q)
            wa[q] = ((pick(ga[q]) & keep) | unit) >> (8 * shalf);
#pragma unroll
        for (int q = 0; q < TN; ++q)
            wb[q] = ((pick(gb[q]) & keep) | unit) >> (8 * shalf);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            i32x8 fa[TM], fb[TN];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int q = 0; q < TM; ++q) {
                    const i32x4 v = *reinterpret_cast<const i32x4 *>(st + a_lane[kk][half] + q * 32 * BKB);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        fa[q][4 * half + e] = v[e];
                }
#pragma unroll
                for (int q = 0; q < TN; ++q) {
                    const i32x4 v = *reinterpret_cast<const i32x4 *>(st + b_lane[kk][half] + q * 32 * BKB);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        fb[q][4 * half + e] = v[e];
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if (kk == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[j], fa[i], acc[i][j], MX_FMT_B(FMT), MX_FMT_A(FMT), 0, (int)wb[j], 0,
                            (int)wa[i]);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[j], fa[i], acc[i][j], MX_FMT_B(FMT), MX_FMT_A(FMT), 2, (int)wb[j], 2,
                            (int)wa[i]);
                }
        }
    }
    wait_vmem<0>();  // the trailing empty DMAs still write their stages
    barrier_lds();   // every wave is done with the stages before they hold D

    // staged epilogue, as in gemm_dma_kernel
    constexpr int SROW = WTN;
    constexpr int SCH = WTN / 8;
    static_assert((SCH & (SCH - 1)) == 0 && SCH >= 2, "chunk swizzle needs a power of two");
    auto stage_off = [](int r, int chunk) { return r * SROW + ((chunk ^ (r & (SCH - 1))) << 3); };
    E *stg = reinterpret_cast<E *>(smem) + wave * WTM * WTN;
    const int frag_row = frag_row_of(lane), frag_hi = frag_hi_of(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                V4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (E)acc[i][j][g * 4 + r];  // round to nearest even
                const int r = i * 32 + frag_row;
                const int c = j * 32 + g * 8 + frag_hi * 4;
                *reinterpret_cast<V4 *>(stg + stage_off(r, c / 8) + (c & 7)) = h;
            }
        store_staged_block<E, WTM, WTN, decltype(stage_off), 32>(stg, stage_off, D, ldd, m0, n0 + wave * WTN, M,
                                                                 N, dvec, lane, 32 * i);
    }
}

struct KernelChoice {
    const void *fn;
    const char *tile;  // "<BM>x<BN>_w<WM>x<WN>"
    int bm, bn, threads;
    int path;
    bool persistent = false;  // grid: one workgroup per compute unit, not one per tile
};

// Compile-time tuning of the direct-to-LDS kernels: K-tile depth (BK), LDS
// ring depth (STAGES) and DMA spread per workgroup tile size (M: 128×128,
// S: 64×64, K*: column strips; the 256×256 tile uses gemm_dma3_kernel).
// The defaults are the measured best on MI355X.
#ifndef TG_M_DMA_STEPS
#define TG_M_DMA_STEPS 2
#endif
#ifndef TG_S_DMA_STEPS
#define TG_S_DMA_STEPS 2
#endif
#ifndef TG_M_BK
#define TG_M_BK 64
#endif
#ifndef TG_M_STAGES
#define TG_M_STAGES 4
#endif
// The 64×64 tile takes 128-K tiles in three stages (32 KiB each): its small
// MFMA work per K-tile left the K loop bound by the per-K-tile wait and
// barrier, and halving their number measured 4–11% faster than 64-K tiles
// in four stages (64×3584×8192 30.3 → 26.9 µs, 32×4096×4096 16.4 → 14.8,
// 1000²×4096 19.3 → 17.2, 1000³ 6.94 → 6.65, 1024³ 6.45 → 6.12; one box),
// while deeper 64-K rings (6–10 stages) measured no better.
#ifndef TG_S_BK
#define TG_S_BK 128
#endif
#ifndef TG_S_STAGES
#define TG_S_STAGES 3
#endif
#ifndef TG_S_KROT
#define TG_S_KROT 0
#endif
#ifndef TG_M_KROT
#define TG_M_KROT 0
#endif
// MFMA shape per tile (16: v_mfma_f32_16x16x32, 32: v_mfma_f32_32x32x16).
// The 64×64 tile runs faster with the 16×16 shape (10–15% on 1000³, 1024³,
// 512×512×4096); the 128×128 tile measured mixed (−5% to +2%), so keeps 32.
// Producer/consumer 128×128 kernel in place of the 128×128 one on the
// direct-to-LDS path (1) or not (0), and its LDS stages.  Measured on one
// box (steady state): 2048×2048×4096 43.2 → 34.4 µs, 2048×4096×4096 81.5 →
// 65.4, 1536×3072×4096 63.1 → 53.7, 2560³ 48.6 → 41.6, 3072²×1024 32.9 →
// 29.5, 2048³ 22.1 → 20.9; three, four or five stages within 2%.
#ifndef TG_WS_ON
#define TG_WS_ON 1
#endif
#ifndef TG_WS_STAGES
#define TG_WS_STAGES 4
#endif
#ifndef TG_M_MF
#define TG_M_MF 32
#endif
#ifndef TG_S_MF
#define TG_S_MF 16
#endif

// Persistent 256×256 kernel: stages of A (3: A three, B two; 2: the
// reverse), tile rows per group of the tile order, fragment-read spacing of
// the K-step before the barrier, and the tiles per compute unit from which
// it replaces the one-tile-per-workgroup launch (0: never).
#ifndef TG_P_SA
#define TG_P_SA 3
#endif
#ifndef TG_P_GM
#define TG_P_GM 4
#endif
#ifndef TG_P_RS0
#define TG_P_RS0 4
#endif
#ifndef TG_P_MIN_PER_CU
#define TG_P_MIN_PER_CU 2
#endif

// Tiles of 256×256 from which that tile replaces the 128×128 one (5/8 of
// the compute units).
#ifndef TG_L_MIN_TILES
#define TG_L_MIN_TILES (5 * NUM_CU / 8)
#endif

// MFMA shape of the 256×256 kernel: 16 (v_mfma_f32_16x16x32, the default:
// the same work in twice the instructions draws less power, so the clock
// holds higher under load) or 32 (v_mfma_f32_32x32x16).
#ifndef TG_L_MF
#define TG_L_MF 16
#endif

// Load path of a launch: direct-to-LDS DMA, 16-byte loads through registers
// (aligned operands whose in-tile offsets exceed 32 bits), or element-wise.
enum LoadPath { PATH_DMA = 0, PATH_VEC = 1, PATH_SCALAR = 2 };

template <typename E, int BM, int BN, int WM, int WN, int DMA_BK, int DMA_STAGES,
          int DMA_STEPS = 1, int OCC = 1, int KROT = 0, int MF = 32>
KernelChoice choice(LoadPath path, const char *tile)
{
    const void *fn =
        path == PATH_DMA
            ? reinterpret_cast<const void *>(
                  &gemm_dma_kernel<E, BM, BN, WM, WN, DMA_BK, DMA_STAGES, OCC, DMA_STEPS, KROT, MF>)
        : path == PATH_VEC ? reinterpret_cast<const void *>(&gemm_vec_kernel<E, BM, BN, WM, WN, true>)
                           : reinterpret_cast<const void *>(&gemm_vec_kernel<E, BM, BN, WM, WN, false>);
    return {fn, tile, BM, BN, WM * WN * 64, path};
}

constexpr const char *PATH_SUFFIX[3] = {"_dma", "_vec", "_scalar"};
#define TG_STR2(x) #x
#define TG_STR(x) TG_STR2(x)
#define TG_TILE(bm, bn, wm, wn) TG_STR(bm) "x" TG_STR(bn) "_w" TG_STR(wm) "x" TG_STR(wn)
// Column-strip tiles for small M: one tile row covers all of M.
#ifndef TG_K_BN
#define TG_K_BN 128
#endif
#ifndef TG_K_WN
#define TG_K_WN 4
#endif
#ifndef TG_K_STAGES
#define TG_K_STAGES 4
#endif
#ifndef TG_K_BK
#define TG_K_BK 64
#endif
#ifndef TG_K_DS
#define TG_K_DS 2
#endif
#ifndef TG_K_ON
#define TG_K_ON 1
#endif
#ifndef TG_K2_STAGES
#define TG_K2_STAGES 4
#endif
#ifndef TG_K2_BK
#define TG_K2_BK 64
#endif
#ifndef TG_K4_STAGES
#define TG_K4_STAGES 3
#endif
#ifndef TG_K4_BK
#define TG_K4_BK 64
#endif
#ifndef TG_K_MAXM
#define TG_K_MAXM 256
#endif
constexpr const char *TILE_STRIP64 = TG_TILE(64, TG_K_BN, 1, TG_K_WN);
// The 128×128 column strip shares its tile and wave grid with the general
// 128×128 tile; its name says "strip" so that the two instantiations (K
// rotation and streaming B here) stay apart in plans and profiles.
constexpr const char *TILE_STRIP128 = TG_TILE(128, 128, 2, 2) "_strip";
constexpr const char *TILE_STRIP256 = TG_TILE(256, 128, 2, 2);
constexpr const char *TILE_256 = TG_TILE(256, 256, 2, 2);
constexpr const char *TILE_256P = TG_TILE(256, 256, 2, 2) "_pers";
constexpr const char *TILE_128 = TG_TILE(128, 128, 2, 2);
constexpr const char *TILE_128WS = TG_TILE(128, 128, 2, 2) "_ws";
constexpr const char *TILE_64 = TG_TILE(64, 64, 2, 2);
constexpr const char *TILE_6432 = TG_TILE(64, 32, 2, 2);
// 64×32 tiles in place of 64×64 ones on the direct-to-LDS path when there are
// at most TG_N_MAX_TILES of the latter and K is at least TG_N_MIN_K: with so
// few tiles each workgroup is bound by the operand bytes its DMAs bring in
// per K-tile, and every workgroup reads all 64 rows of A; halving the B rows
// cuts that by a quarter and doubles the workgroups (6–9% faster on
// 64×3584×8192, 64×7168×8192, 128×3584×8192, 32×4096², 64×2048×16384,
// 256×512×8192, 512²×4096, 100×1000×2048; one box).
#ifndef TG_N_MAX_TILES
#define TG_N_MAX_TILES 128
#endif
#ifndef TG_N_MIN_K
#define TG_N_MIN_K 2048
#endif

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

// D store mode of a staged epilogue (2-byte elements): 16-byte stores when
// every row is 16-byte aligned, non-temporal from D_NT_MIN_BYTES of D on
// when a 256-row block's byte offsets fit the stores' 32-bit offsets.
constexpr int64_t D_NT_MIN_BYTES = 4 << 20;
int d_store_mode(const void *D, int64_t M, int64_t N, int64_t ldd)
{
    if (ldd % 8 != 0 || (uintptr_t)D % 16 != 0)
        return D_ELEM;
    return M * N * 2 >= D_NT_MIN_BYTES && 256 * ldd * 2 + 512 < (int64_t)DMA_RANGE ? D_VEC_NT : D_VEC;
}

struct Plan {
    KernelChoice k;
    int tiles_m, tiles_n;
    int dvec;
};

template <typename E>
Plan make_plan(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldd)
{
    const bool vec = (K % 8 == 0) && (lda % 8 == 0) && (ldb % 8 == 0) &&
                     ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
    const auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const auto path = [&](int bm, int bn) {
        if (!vec)
            return PATH_SCALAR;
        return dma_offsets_fit(bm, lda) && dma_offsets_fit(bn, ldb) ? PATH_DMA : PATH_VEC;
    };
    KernelChoice k;
    // Small M, large N (HBM-bound streaming of B): one tile row covers all of
    // M, so B is read exactly once, and the XCDs start at spread K offsets.
    if (TG_K_ON && M <= 64 && tiles(64, TG_K_BN) >= NUM_CU / 2)
        k = choice<E, 64, TG_K_BN, 1, TG_K_WN, TG_K_BK, TG_K_STAGES, TG_K_DS, 1, 1>(
            path(64, TG_K_BN), TILE_STRIP64);
    else if (TG_K_ON && M <= 128 && TG_K_MAXM >= 128 && tiles(128, 128) >= NUM_CU / 2)
        k = choice<E, 128, 128, 2, 2, TG_K2_BK, TG_K2_STAGES, 2, 1, 1>(
            path(128, 128), TILE_STRIP128);
    else if (TG_K_ON && M <= 256 && TG_K_MAXM >= 256 && tiles(256, 128) >= NUM_CU / 2)
        k = choice<E, 256, 128, 2, 2, TG_K4_BK, TG_K4_STAGES, 2, 1, 1>(path(256, 128), TILE_STRIP256);
    else
    // the 256×256 kernel from 160 tiles on (5/8 of the CUs busy): it beats
    // the 128×128 tiles by 20–40% at 160–224 tiles (the 128×128 grid then
    // runs 2.5–3.5 waves); at 128 tiles (exactly two waves of 128×128) the
    // smaller tile is 5–9% faster
    if (tiles(256, 256) >= TG_L_MIN_TILES) {
        const LoadPath lp = path(256, 256);
        // several tiles per compute unit and whole K-tiles: the persistent form
        if (lp == PATH_DMA && TG_P_MIN_PER_CU > 0 && tiles(256, 256) >= TG_P_MIN_PER_CU * NUM_CU &&
            K >= 128 && K % 64 == 0) {
            k = {reinterpret_cast<const void *>(&gemm_pers_kernel<E, TG_P_SA, TG_P_GM, TG_P_RS0>), TILE_256P,
                 256, 256, 256, PATH_DMA, true};
        } else if (lp == PATH_DMA)
            k = {reinterpret_cast<const void *>(&gemm_dma3_kernel<E, 256, 256, 2, 2, TG_L_MF>), TILE_256, 256,
                 256, 256, PATH_DMA};
        else
            k = choice<E, 256, 256, 2, 2, 64, 2>(lp, TILE_256);
    }
    // 128×128 tiles from 80 of them on: at 81–224 tiles they beat the 64×64
    // grid by 15–90% (1152²×1024, 1024×1536×4096, 2048×1280×4096,
    // 1792×2048×2048); at 48–64 (1000³, 1024²×4096, 768×1024×4096) the
    // 64×64 grid is faster
    else if (tiles(128, 128) >= 5 * NUM_CU / 16) {
        const LoadPath lp = path(128, 128);
        if (lp == PATH_DMA && TG_WS_ON)
            k = {reinterpret_cast<const void *>(&gemm_ws_kernel<E, TG_WS_STAGES>), TILE_128WS, 128, 128, 512,
                 PATH_DMA};
        else
            k = choice<E, 128, 128, 2, 2, TG_M_BK, TG_M_STAGES, TG_M_DMA_STEPS, 1, TG_M_KROT, TG_M_MF>(
                lp, TILE_128);
    }
    else if (tiles(64, 64) <= TG_N_MAX_TILES && K >= TG_N_MIN_K && path(64, 32) == PATH_DMA)
        k = {reinterpret_cast<const void *>(
                 &gemm_dma_kernel<E, 64, 32, 2, 2, TG_S_BK, TG_S_STAGES, 1, TG_S_DMA_STEPS, 0, TG_S_MF>),
             TILE_6432, 64, 32, 256, PATH_DMA};
    else
        k = choice<E, 64, 64, 2, 2, TG_S_BK, TG_S_STAGES, TG_S_DMA_STEPS, 1, TG_S_KROT, TG_S_MF>(
            path(64, 64), TILE_64);
    Plan p;
    p.k = k;
    p.tiles_m = (int)((M + k.bm - 1) / k.bm);
    p.tiles_n = (int)((N + k.bn - 1) / k.bn);
    // vector stores: 16 bytes (staged epilogue of the DMA kernels; non-
    // temporal for a large D) or 8 bytes
    p.dvec = p.k.path == PATH_DMA ? d_store_mode(D, M, N, ldd) : (ldd % 4 == 0) && ((uintptr_t)D % 8 == 0);
    return p;
}

// per-device "is gfx950" cache: 0 unknown, 1 yes, -1 no
std::atomic<int> g_arch_ok[64];
// per-device compute-unit count (0: not yet queried)
std::atomic<int> g_cus[64];

// Workgroups of a persistent launch: one per compute unit, rounded down to a
// multiple of the 8 XCDs (workgroup w runs on XCD w mod 8, and the tile order
// keeps each XCD's tiles together), never more than there are tiles.
int64_t persistent_grid(int64_t tiles)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64)
        cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = NUM_CU;
        if (dev >= 0 && dev < 64)
            g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    int64_t g = (int64_t)cus / NUM_XCD * NUM_XCD;
    if (g < NUM_XCD)
        g = NUM_XCD;
    return g < tiles ? g : tiles;
}

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

template <typename E>
int launch(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, int64_t lda,
           int64_t ldb, int64_t ldd, void *stream)
{
    int st = validate(A, B, D, M, N, K, lda, ldb, ldd);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_OK;
    st = check_device();
    if (st != TG_OK)
        return st;
    Plan p = make_plan<E>(A, B, D, M, N, K, lda, ldb, ldd);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    const int64_t grid = p.k.persistent ? persistent_grid(tiles) : tiles;
    int Mi = (int)M, Ni = (int)N, Ki = (int)K;
    unsigned long long *no_stamps = nullptr;  // the persistent kernel's last argument; others take 12
    void *args[] = {(void *)&A, (void *)&B, (void *)&D, &Mi, &Ni, &Ki, &lda, &ldb, &ldd,
                    &p.tiles_m, &p.tiles_n, &p.dvec, &no_stamps};
    hipError_t e = hipLaunchKernel(p.k.fn, dim3((unsigned)grid), dim3(p.k.threads), args, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

// The fp16 GEMM through the stamping instantiation of the persistent kernel
// (measurement only): the plan must be the persistent one, and `stamps`
// must hold three words per workgroup.
int launch_stamped(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, int64_t lda,
                   int64_t ldb, int64_t ldd, uint64_t *stamps, int64_t stamps_len, int64_t *workgroups,
                   void *stream)
{
    if (workgroups)
        *workgroups = 0;
    int st = validate(A, B, D, M, N, K, lda, ldb, ldd);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_ERR_INVALID_ARG;
    Plan p = make_plan<_Float16>(A, B, D, M, N, K, lda, ldb, ldd);
    if (!p.k.persistent)
        return TG_ERR_INVALID_ARG;
    const int64_t grid = persistent_grid((int64_t)p.tiles_m * p.tiles_n);
    if (!stamps || stamps_len < 3 * grid)
        return TG_ERR_INVALID_ARG;
    st = check_device();
    if (st != TG_OK)
        return st;
    if (workgroups)
        *workgroups = grid;
    int Mi = (int)M, Ni = (int)N, Ki = (int)K;
    unsigned long long *sp = reinterpret_cast<unsigned long long *>(stamps);
    void *args[] = {(void *)&A, (void *)&B, (void *)&D, &Mi, &Ni, &Ki, &lda, &ldb, &ldd,
                    &p.tiles_m, &p.tiles_n, &p.dvec, &sp};
    const void *fn = reinterpret_cast<const void *>(&gemm_pers_kernel<_Float16, TG_P_SA, TG_P_GM, TG_P_RS0, true>);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

template <typename E>
int plan(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K,
         int64_t lda, int64_t ldb, int64_t ldd, char *name, int64_t name_len, int64_t *tiles)
{
    int st = validate(A, B, D, M, N, K, lda, ldb, ldd);
    if (name && name_len > 0)
        name[0] = 0;
    if (tiles)
        *tiles = 0;
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    Plan p = make_plan<E>(A, B, D, M, N, K, lda, ldb, ldd);
    if (name && name_len > 0)
        snprintf(name, (size_t)name_len, "%s%s%s", Elem<E>::prefix, p.k.tile, PATH_SUFFIX[p.k.path]);
    if (tiles)
        *tiles = (int64_t)p.tiles_m * p.tiles_n;
    return TG_OK;
}

}  // namespace

extern "C" int tg_gemm_f16(const void *A, const void *B, void *D, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldd, void *stream)
{
    return launch<_Float16>(A, B, D, M, N, K, lda, ldb, ldd, stream);
}

extern "C" int tg_gemm_f16_xcd_stamps(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                                      int64_t lda, int64_t ldb, int64_t ldd, uint64_t *stamps, int64_t stamps_len,
                                      int64_t *workgroups, void *stream)
{
    return launch_stamped(A, B, D, M, N, K, lda, ldb, ldd, stamps, stamps_len, workgroups, stream);
}

extern "C" int tg_gemm_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N,
                            int64_t K, int64_t lda, int64_t ldb, int64_t ldd, void *stream)
{
    return launch<__bf16>(A, B, D, M, N, K, lda, ldb, ldd, stream);
}

extern "C" int tg_gemm_f16_plan(const void *A, const void *B, const void *D, int64_t M,
                                int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                                char *name, int64_t name_len, int64_t *tiles)
{
    return plan<_Float16>(A, B, D, M, N, K, lda, ldb, ldd, name, name_len, tiles);
}

extern "C" int tg_gemm_bf16_plan(const void *A, const void *B, const void *D, int64_t M,
                                 int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                                 char *name, int64_t name_len, int64_t *tiles)
{
    return plan<__bf16>(A, B, D, M, N, K, lda, ldb, ldd, name, name_len, tiles);
}

// Block-scaled FP8 entry point: argument checks, then one 256×256 tile per
// workgroup, or one 64×128 tile per workgroup where M <= 64 and N gives at
// least 128 column strips (HBM-bound: B streams once) or where the problem
// has too few 256×256 tiles to occupy a quarter of the GPU.
// The 256×256 kernel loads scale words in groups of four K-tiles when four
// divide the K-tile count, else in pairs: two instantiations, two names.
namespace {

constexpr const char *MXF8_KERNEL_G4 = "gemm_mxf8_256x256_w2x2_g4_dma";
constexpr const char *MXF8_KERNEL_G2 = "gemm_mxf8_256x256_w2x2_g2_dma";
constexpr const char *MXF8_STRIP_KERNEL = "gemm_mxf8_64x128_w1x4_dma";
// the same kernels reading scales in the packed layout
constexpr const char *MXF8P_KERNEL_G4 = "gemm_mxf8p_256x256_w2x2_g4_dma";
constexpr const char *MXF8P_KERNEL_G2 = "gemm_mxf8p_256x256_w2x2_g2_dma";
constexpr const char *MXF8P_STRIP_KERNEL = "gemm_mxf8p_64x128_w1x4_dma";
#ifndef TG_MX_STRIP_STAGES
#define TG_MX_STRIP_STAGES 4
#endif
bool mx_group4(int64_t K) { return ((K + 127) / 128) % 4 == 0; }
bool mx_uses_strip(int64_t M, int64_t N)
{
    return (M <= 64 && (N + 127) / 128 >= NUM_CU / 2) || ((M + 255) / 256) * ((N + 255) / 256) < NUM_CU / 4;
}
int64_t mx_strip_tiles(int64_t M, int64_t N) { return ((M + 63) / 64) * ((N + 127) / 128); }

int validate_mx(const void *A, const void *SA, const void *B, const void *SB, const void *D, int64_t M,
                int64_t N, int64_t K, int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldd < N || ldsa < (K + 31) / 32 ||
        ldsb < (K + 31) / 32 || lda < 0 || ldb < 0 || ldsa < 0 || ldsb < 0 || ldd < 0)
        return TG_ERR_INVALID_ARG;
    if ((M > 0 && K > 0 && (!A || !SA)) || (N > 0 && K > 0 && (!B || !SB)) || (M > 0 && N > 0 && !D))
        return TG_ERR_INVALID_ARG;
    if (M >= LIMIT32 || N >= LIMIT32 || K >= LIMIT32 || lda >= LIMIT32 || ldb >= LIMIT32 ||
        ldd >= LIMIT32 || 255 * lda + 128 >= DMA_RANGE || 255 * ldb + 128 >= DMA_RANGE ||
        256 * ldsa + 4 * K >= LIMIT32 || 256 * ldsb + 4 * K >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    if (K % 32 != 0 || lda % 16 != 0 || ldb % 16 != 0 || ldsa % 4 != 0 || ldsb % 4 != 0 ||
        (uintptr_t)A % 16 != 0 || (uintptr_t)B % 16 != 0 || (uintptr_t)SA % 4 != 0 || (uintptr_t)SB % 4 != 0)
        return TG_ERR_LAYOUT;
    return TG_OK;
}

// Bytes of one 32-row group of the packed scale layout: 512 per 16 blocks
// (512 elements) of K.
int64_t mx_packed_stride(int64_t K) { return (K + 511) / 512 * 512; }

int validate_mx_packed(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                       int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldd < N)
        return TG_ERR_INVALID_ARG;
    if ((M > 0 && K > 0 && (!A || !SA)) || (N > 0 && K > 0 && (!B || !SB)) || (M > 0 && N > 0 && !D))
        return TG_ERR_INVALID_ARG;
    if (M >= LIMIT32 || N >= LIMIT32 || K >= LIMIT32 || lda >= LIMIT32 || ldb >= LIMIT32 ||
        ldd >= LIMIT32 || 255 * lda + 128 >= DMA_RANGE || 255 * ldb + 128 >= DMA_RANGE ||
        K >= ((int64_t)1 << 27))  // packed offsets in a workgroup's rows: < 9·K + 1024
        return TG_ERR_TOO_LARGE;
    if (K % 32 != 0 || lda % 16 != 0 || ldb % 16 != 0 || (uintptr_t)A % 16 != 0 || (uintptr_t)B % 16 != 0 ||
        (uintptr_t)SA % 16 != 0 || (uintptr_t)SB % 16 != 0)
        return TG_ERR_LAYOUT;
    return TG_OK;
}

// Name suffix of the element encodings FMT (none for E4M3 on both operands).
const char *mx_fmt_suffix(int fmt)
{
    return fmt == 1 ? "_e5m2xe4m3" : fmt == 2 ? "_e4m3xe5m2" : fmt == 3 ? "_e5m2" : "";
}

// The kernel a validated block-scaled problem runs on, and its workgroup count.
const char *mx_kernel_name(int64_t M, int64_t N, int64_t K, bool packed)
{
    if (mx_uses_strip(M, N))
        return packed ? MXF8P_STRIP_KERNEL : MXF8_STRIP_KERNEL;
    if (mx_group4(K))
        return packed ? MXF8P_KERNEL_G4 : MXF8_KERNEL_G4;
    return packed ? MXF8P_KERNEL_G2 : MXF8_KERNEL_G2;
}
int64_t mx_tiles(int64_t M, int64_t N)
{
    return mx_uses_strip(M, N) ? mx_strip_tiles(M, N) : ((M + 255) / 256) * ((N + 255) / 256);
}

// The instantiations of the element encodings FMT (0..3).
template <bool PK, int G>
const void *mx_kernel_fn(int fmt)
{
    switch (fmt) {
    case 1:
        return reinterpret_cast<const void *>(&gemm_mxf8_kernel<256, 256, 2, 2, G, PK, 1>);
    case 2:
        return reinterpret_cast<const void *>(&gemm_mxf8_kernel<256, 256, 2, 2, G, PK, 2>);
    case 3:
        return reinterpret_cast<const void *>(&gemm_mxf8_kernel<256, 256, 2, 2, G, PK, 3>);
    default:
        return reinterpret_cast<const void *>(&gemm_mxf8_kernel<256, 256, 2, 2, G, PK, 0>);
    }
}
template <bool PK>
const void *mx_strip_fn(int fmt)
{
    switch (fmt) {
    case 1:
        return reinterpret_cast<const void *>(&gemm_mxf8_strip_kernel<TG_MX_STRIP_STAGES, PK, 1>);
    case 2:
        return reinterpret_cast<const void *>(&gemm_mxf8_strip_kernel<TG_MX_STRIP_STAGES, PK, 2>);
    case 3:
        return reinterpret_cast<const void *>(&gemm_mxf8_strip_kernel<TG_MX_STRIP_STAGES, PK, 3>);
    default:
        return reinterpret_cast<const void *>(&gemm_mxf8_strip_kernel<TG_MX_STRIP_STAGES, PK, 0>);
    }
}

// Launch a validated, non-empty block-scaled problem; lds is the row stride
// (row-major) or the 32-row group stride (packed) of each scale matrix; fmt
// the element encodings (FMT above).
template <bool PK>
int launch_mx(const void *A, const void *SA, const void *B, const void *SB, void *D, int64_t M, int64_t N,
              int64_t K, int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd, int fmt, void *stream)
{
    int st = check_device();
    if (st != TG_OK)
        return st;
    int Mi = (int)M, Ni = (int)N, Ki = (int)K;
    int dvec = d_store_mode(D, M, N, ldd);
    if (mx_uses_strip(M, N)) {
        const int64_t sgrid = mx_strip_tiles(M, N);
        if (sgrid >= LIMIT32)
            return TG_ERR_TOO_LARGE;
        int stiles_n = (int)((N + 127) / 128);
        void *sargs[] = {(void *)&A, (void *)&SA, (void *)&B, (void *)&SB, (void *)&D, &Mi, &Ni, &Ki,
                         &lda, &ldsa, &ldb, &ldsb, &ldd, &stiles_n, &dvec};
        hipError_t e = hipLaunchKernel(mx_strip_fn<PK>(fmt), dim3((unsigned)sgrid), dim3(256), sargs, 0,
                                       (hipStream_t)stream);
        return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
    }
    int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
    const int64_t grid = (int64_t)tiles_m * tiles_n;
    if (grid >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    void *args[] = {(void *)&A, (void *)&SA, (void *)&B, (void *)&SB, (void *)&D, &Mi, &Ni, &Ki,
                    &lda, &ldsa, &ldb, &ldsb, &ldd, &tiles_m, &tiles_n, &dvec};
    // groups of four K-tiles when they divide the K-tile count, else pairs
    // (at most one padding K-tile)
    const void *fn = mx_group4(K) ? mx_kernel_fn<PK, 4>(fmt) : mx_kernel_fn<PK, 2>(fmt);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

void mx_plan_out(const char *kernel, int64_t tiles, char *name, int64_t name_len, int64_t *tiles_out,
                 int fmt = 0)
{
    if (name && name_len > 0)
        snprintf(name, (size_t)name_len, "%s%s", kernel, kernel[0] ? mx_fmt_suffix(fmt) : "");
    if (tiles_out)
        *tiles_out = tiles;
}

// Pack row-major scale bytes (rows × nb blocks, row stride lds) into the
// packed layout: thread i writes the 16 bytes at 16·i, row (i / 32 / nbg)·32
// + i % 32, blocks 16·((i / 32) % nbg) .. +15; bytes outside the matrix get
// E8M0 127 (2^0).
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint8_t *__restrict__ S, int64_t lds, int64_t rows,
                                                      int64_t nb, int64_t nbg, int64_t total,
                                                      uint8_t *__restrict__ P)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total)
        return;
    const int64_t rr = i % 32, g = (i / 32) % nbg, rg = i / (32 * nbg);
    const int64_t row = rg * 32 + rr;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        unsigned v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t blk = g * 16 + 4 * w + b;
            const unsigned byte = row < rows && blk < nb ? S[row * lds + blk] : 127u;
            v |= byte << (8 * b);
        }
        out[w] = v;
    }
    *reinterpret_cast<u32x4 *>(P + 16 * i) = out;
}

}  // namespace

extern "C" int64_t tg_mx_packed_bytes(int64_t rows, int64_t K)
{
    if (rows < 0 || K < 0 || K % 32 != 0 || rows >= LIMIT32 || K >= LIMIT32)
        return -1;
    return (rows + 31) / 32 * mx_packed_stride(K);
}

extern "C" int tg_mx_pack_scales(const void *S, int64_t rows, int64_t K, int64_t lds, void *P, void *stream)
{
    if (rows < 0 || K < 0 || K % 32 != 0 || lds < K / 32 || (rows > 0 && K > 0 && (!S || !P)))
        return TG_ERR_INVALID_ARG;
    if (rows >= LIMIT32 || K >= LIMIT32 || lds >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    if ((uintptr_t)P % 16 != 0)
        return TG_ERR_LAYOUT;
    if (rows == 0 || K == 0)
        return TG_OK;
    const int st = check_device();
    if (st != TG_OK)
        return st;
    const int64_t nb = K / 32, nbg = mx_packed_stride(K) / 512, total = (rows + 31) / 32 * nbg * 32;
    const int64_t grid = (total + 255) / 256;
    if (grid >= LIMIT32)
        return TG_ERR_TOO_LARGE;
    const uint8_t *s = static_cast<const uint8_t *>(S);
    uint8_t *p = static_cast<uint8_t *>(P);
    int64_t lds_ = lds, rows_ = rows;
    void *args[] = {(void *)&s, &lds_, &rows_, (void *)&nb, (void *)&nbg, (void *)&total, (void *)&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&mx_pack_kernel), dim3((unsigned)grid), dim3(256),
                                   args, 0, (hipStream_t)stream);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

// Element encodings of the block-scaled entry points: 0 E4M3, 1 E5M2.
static int mx_fmt(int a_format, int b_format)
{
    if (a_format < 0 || a_format > 1 || b_format < 0 || b_format > 1)
        return -1;
    return a_format + 2 * b_format;
}

extern "C" int tg_gemm_mx(const void *A, const void *SA, const void *B, const void *SB, void *D, int64_t M,
                          int64_t N, int64_t K, int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd,
                          int a_format, int b_format, void *stream)
{
    const int fmt = mx_fmt(a_format, b_format);
    if (fmt < 0)
        return TG_ERR_INVALID_ARG;
    int st = validate_mx(A, SA, B, SB, D, M, N, K, lda, ldsa, ldb, ldsb, ldd);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_OK;
    return launch_mx<false>(A, SA, B, SB, D, M, N, K, lda, ldsa, ldb, ldsb, ldd, fmt, stream);
}

extern "C" int tg_gemm_mx_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldsa, int64_t ldb,
                               int64_t ldsb, int64_t ldd, int a_format, int b_format, char *name,
                               int64_t name_len, int64_t *tiles)
{
    const int fmt = mx_fmt(a_format, b_format);
    mx_plan_out("", 0, name, name_len, tiles);
    if (fmt < 0)
        return TG_ERR_INVALID_ARG;
    int st = validate_mx(A, SA, B, SB, D, M, N, K, lda, ldsa, ldb, ldsb, ldd);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    mx_plan_out(mx_kernel_name(M, N, K, false), mx_tiles(M, N), name, name_len, tiles, fmt);
    return TG_OK;
}

extern "C" int tg_gemm_mx_packed(const void *A, const void *SA, const void *B, const void *SB, void *D, int64_t M,
                                 int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd, int a_format,
                                 int b_format, void *stream)
{
    const int fmt = mx_fmt(a_format, b_format);
    if (fmt < 0)
        return TG_ERR_INVALID_ARG;
    int st = validate_mx_packed(A, SA, B, SB, D, M, N, K, lda, ldb, ldd);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_OK;
    const int64_t stride = mx_packed_stride(K);
    return launch_mx<true>(A, SA, B, SB, D, M, N, K, lda, stride, ldb, stride, ldd, fmt, stream);
}

extern "C" int tg_gemm_mx_packed_plan(const void *A, const void *SA, const void *B, const void *SB, const void *D,
                                      int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                                      int a_format, int b_format, char *name, int64_t name_len, int64_t *tiles)
{
    const int fmt = mx_fmt(a_format, b_format);
    mx_plan_out("", 0, name, name_len, tiles);
    if (fmt < 0)
        return TG_ERR_INVALID_ARG;
    int st = validate_mx_packed(A, SA, B, SB, D, M, N, K, lda, ldb, ldd);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    mx_plan_out(mx_kernel_name(M, N, K, true), mx_tiles(M, N), name, name_len, tiles, fmt);
    return TG_OK;
}

// E4M3 on both operands
extern "C" int tg_gemm_mxf8(const void *A, const void *SA, const void *B, const void *SB, void *D,
                            int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldsa, int64_t ldb,
                            int64_t ldsb, int64_t ldd, void *stream)
{
    return tg_gemm_mx(A, SA, B, SB, D, M, N, K, lda, ldsa, ldb, ldsb, ldd, 0, 0, stream);
}

extern "C" int tg_gemm_mxf8_plan(const void *A, const void *SA, const void *B, const void *SB,
                                 const void *D, int64_t M, int64_t N, int64_t K, int64_t lda,
                                 int64_t ldsa, int64_t ldb, int64_t ldsb, int64_t ldd, char *name,
                                 int64_t name_len, int64_t *tiles)
{
    return tg_gemm_mx_plan(A, SA, B, SB, D, M, N, K, lda, ldsa, ldb, ldsb, ldd, 0, 0, name, name_len, tiles);
}

extern "C" int tg_gemm_mxf8_packed(const void *A, const void *SA, const void *B, const void *SB, void *D,
                                   int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldd,
                                   void *stream)
{
    return tg_gemm_mx_packed(A, SA, B, SB, D, M, N, K, lda, ldb, ldd, 0, 0, stream);
}

extern "C" int tg_gemm_mxf8_packed_plan(const void *A, const void *SA, const void *B, const void *SB,
                                        const void *D, int64_t M, int64_t N, int64_t K, int64_t lda,
                                        int64_t ldb, int64_t ldd, char *name, int64_t name_len, int64_t *tiles)
{
    return tg_gemm_mx_packed_plan(A, SA, B, SB, D, M, N, K, lda, ldb, ldd, 0, 0, name, name_len, tiles);
}

extern "C" int tg_device_info(int *compute_units, int *max_clock_khz, char *arch, int64_t arch_len)
{
    int dev = 0, cus = 0, clk = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return TG_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, dev) != hipSuccess ||
        hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return TG_ERR_DEVICE;
    if (compute_units)
        *compute_units = cus;
    if (max_clock_khz)
        *max_clock_khz = clk;
    if (arch && arch_len > 0)
        snprintf(arch, (size_t)arch_len, "%s", prop.gcnArchName);
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
    case TG_ERR_LAYOUT:
        return "block-scaled layout not supported (K % 32, lda/ldb % 16, ldsa/ldsb % 4, or alignment)";
    default:
        return "unknown status";
    }
}
