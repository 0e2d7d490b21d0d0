// tile_layout.hpp — the shard/replica/offset TileLayout model and the XOR
// swizzle composition, as constexpr C++ usable at compile time by the kernels
// and at run time by the host ABI in tile_layout_abi.cpp.
//
// Model ("TIRx Layout API", sections "TileLayout", "组合三个部分", "正向映射",
// "ComposeLayout", "Swizzle 变换"; "TIRx 基础", section "Layout API"):
//   - a layout is a shard spec S[(e0..en-1):(s0@a0 .. sn-1@an-1)], an optional
//     replica spec R[...] of the same form, and a fixed offset O = Σ v@axis;
//   - L(x) = { D(x) + r + O | r in R }: D(x) splits the flat logical index
//     row-major by the shard extents (last extent fastest) into components
//     c_k and adds c_k·s_k to axis a_k; several iters may feed one axis;
//   - apply() returns D(x) + O only; replicas stay in the layout and are
//     enumerated separately;
//   - ComposeLayout(per_element=M, swizzle_len=B, atom_len=S, tile) first
//     evaluates a tile layout that may only produce the linear axis m, then
//     keeps the low M bits of m and XORs bits [S, S+B) of the rest into bits
//     [0, B) (swizzle_inner) — valid only when S >= B.
// Axis names are part of the meaning: 1@laneid and 1@TLane are different
// places.  On CDNA the lane axis runs over 64 lanes and "warpid" is the wave.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TG_HD __host__ __device__
#else
#define TG_HD
#endif

namespace tg {
namespace layout {

enum Axis : int {
    m = 0,
    laneid,
    warpid,
    tx,
    wgid,
    tid_in_wg,
    wid_in_wg,
    bx,
    by,
    bz,
    cbx,
    cby,
    cbz,
    TLane,
    TCol,
    NUM_AXES
};

constexpr const char *axis_name(int a)
{
    constexpr const char *names[NUM_AXES] = {"m",   "laneid", "warpid", "tx",  "wgid",
                                             "tid_in_wg", "wid_in_wg", "bx", "by", "bz",
                                             "cbx", "cby",    "cbz",    "TLane", "TCol"};
    return (a >= 0 && a < NUM_AXES) ? names[a] : "?";
}

constexpr int MAX_ITERS = 12;

struct Iter {
    int64_t extent = 1;
    int64_t stride = 0;
    int axis = m;
};

struct Coord {
    int64_t v[NUM_AXES] = {};
    constexpr int64_t operator[](int a) const { return v[a]; }
    constexpr bool operator==(const Coord &o) const
    {
        for (int a = 0; a < NUM_AXES; ++a)
            if (v[a] != o.v[a])
                return false;
        return true;
    }
};

struct TileLayout {
    Iter shard[MAX_ITERS] = {};
    int n_shard = 0;
    Iter replica[MAX_ITERS] = {};
    int n_replica = 0;
    int64_t offset[NUM_AXES] = {};

    constexpr TileLayout &S(int64_t extent, int64_t stride, int axis = m)
    {
        shard[n_shard++] = Iter{extent, stride, axis};
        return *this;
    }
    constexpr TileLayout &R(int64_t extent, int64_t stride, int axis = m)
    {
        replica[n_replica++] = Iter{extent, stride, axis};
        return *this;
    }
    constexpr TileLayout &O(int64_t value, int axis)
    {
        offset[axis] += value;
        return *this;
    }

    // number of logical elements the shard covers
    constexpr int64_t size() const
    {
        int64_t n = 1;
        for (int k = 0; k < n_shard; ++k)
            n *= shard[k].extent;
        return n;
    }
    constexpr int64_t replica_count() const
    {
        int64_t n = 1;
        for (int k = 0; k < n_replica; ++k)
            n *= replica[k].extent;
        return n;
    }
    // axis a receives a contribution from the shard or the offset
    constexpr bool uses_axis(int a) const
    {
        if (offset[a] != 0)
            return true;
        for (int k = 0; k < n_shard; ++k)
            if (shard[k].axis == a)
                return true;
        return false;
    }

    // apply(*shard_coord): components given directly
    constexpr Coord apply_shard(const int64_t *c) const
    {
        Coord out;
        for (int a = 0; a < NUM_AXES; ++a)
            out.v[a] = offset[a];
        for (int k = 0; k < n_shard; ++k)
            out.v[shard[k].axis] += c[k] * shard[k].stride;
        return out;
    }
    // apply(linear_coord): split row-major by the shard extents
    constexpr Coord apply(int64_t flat) const
    {
        int64_t c[MAX_ITERS] = {};
        for (int k = n_shard - 1; k >= 0; --k) {
            c[k] = flat % shard[k].extent;
            flat /= shard[k].extent;
        }
        return apply_shard(c);
    }
    // apply(*logical_coord, shape=...): flatten row-major with `shape`
    constexpr Coord apply(const int64_t *x, const int64_t *shape, int rank) const
    {
        int64_t flat = 0;
        for (int d = 0; d < rank; ++d)
            flat = flat * shape[d] + x[d];
        return apply(flat);
    }
    constexpr Coord apply2(int64_t i, int64_t j, int64_t cols) const { return apply(i * cols + j); }

    // r-th replica offset (row-major over the replica extents)
    constexpr Coord replica_offset(int64_t r) const
    {
        Coord out;
        for (int k = n_replica - 1; k >= 0; --k) {
            out.v[replica[k].axis] += (r % replica[k].extent) * replica[k].stride;
            r /= replica[k].extent;
        }
        return out;
    }
};

// XOR swizzle on a linear element address ("Swizzle 变换").
struct Swizzle {
    int per_element = 0;  // M: low bits kept
    int swizzle_len = 0;  // B: width of the XOR field
    int atom_len = 0;     // S: distance between the two fields
    bool inner = true;

    constexpr bool valid() const { return atom_len >= swizzle_len && per_element >= 0; }
    constexpr int64_t operator()(int64_t addr) const
    {
        const int64_t mask = (int64_t(1) << swizzle_len) - 1;
        const int64_t low = addr & ((int64_t(1) << per_element) - 1);
        const int64_t x = addr >> per_element;
        // inner: bits [S, S+B) of x into [0, B); mirrored: bits [0, B) into [S, S+B)
        const int64_t x2 = inner ? (x ^ ((x >> atom_len) & mask)) : (x ^ ((x & mask) << atom_len));
        return (x2 << per_element) | low;
    }
};

struct ComposeLayout {
    Swizzle sw;
    TileLayout tile;

    // the tile may only produce the linear axis m
    constexpr bool well_formed() const
    {
        if (!sw.valid())
            return false;
        for (int a = 0; a < NUM_AXES; ++a)
            if (a != m && tile.uses_axis(a))
                return false;
        return true;
    }
    constexpr int64_t apply(int64_t flat) const { return sw(tile.apply(flat)[m]); }
    constexpr int64_t apply2(int64_t i, int64_t j, int64_t cols) const { return apply(i * cols + j); }
};

// ---------------------------------------------------------------- presets

// row-major (rows × cols) tile on the linear axis: S[(rows,cols):(cols@m,1@m)]
constexpr TileLayout row_major(int64_t rows, int64_t cols)
{
    TileLayout t;
    t.S(rows, cols, m).S(cols, 1, m);
    return t;
}

// 128-byte swizzle for fp16 (16-byte vectors, 8 rows of 128 bytes per atom):
// ComposeLayout(3, 3, 3, S[(rows,64):(64@m,1@m)])
constexpr ComposeLayout swizzle128_f16(int64_t rows)
{
    return ComposeLayout{Swizzle{3, 3, 3, true}, row_major(rows, 64)};
}

// Operand-tile swizzle for a (rows × cols) fp16 tile, cols in {16, 32, 64}:
// ComposeLayout(3, log2(cols/8), 4) — 16-byte vectors stay whole and the
// chunk index is XORed with the row bits above one 256-byte line.
constexpr int ilog2(int64_t x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr ComposeLayout swizzle_bank256_f16(int64_t rows, int64_t cols)
{
    return ComposeLayout{Swizzle{3, ilog2(cols / 8), 4, true}, row_major(rows, cols)};
}

// The operand-tile swizzle the kernels use: ComposeLayout(3, 3, 4) over
// S[(rows,64):(64@m,1@m)], i.e. 16-byte chunk c of row r lands at chunk
// c ^ ((r >> 1) & 7).  Same vector-keeping M = 3 as the 128-byte mode, but the
// XOR field comes from the row pair instead of the row: sixteen consecutive
// rows then cover every 16-byte slot of a 256-byte bank line once, which a
// 64-bank LDS serving 16 lanes per 128-bit read needs (the 128-byte mode
// sends rows r and r+8 to the same banks).
constexpr ComposeLayout swizzle_pairs_f16(int64_t rows)
{
    return ComposeLayout{Swizzle{3, 3, 4, true}, row_major(rows, 64)};
}

// Operand fragment of v_mfma_f32_32x32x16_f16 over a logical 32×16 (row, k)
// tile: lane = row + 32·(k / 8), register element = k mod 8, i.e.
// S[(32,2,8):(1@laneid,32@laneid,1@m)].
constexpr TileLayout mfma32x32x16_operand()
{
    TileLayout t;
    t.S(32, 1, laneid).S(2, 32, laneid).S(8, 1, m);
    return t;
}

// Accumulator of v_mfma_f32_32x32x16_f16 over a logical 32×32 (row, col)
// tile: row = 8·(v/4) + 4·(lane/32) + v%4, col = lane % 32, i.e.
// S[(4,2,4,32):(4@m,32@laneid,1@m,1@laneid)].
constexpr TileLayout mfma32x32_acc()
{
    TileLayout t;
    t.S(4, 4, m).S(2, 32, laneid).S(4, 1, m).S(32, 1, laneid);
    return t;
}

// The same accumulator read with the MFMA inputs swapped (the GEMM's B feeds
// the MFMA's first input), over a logical 32×32 tile of D: D row = lane % 32,
// D col = 8·(v/4) + 4·(lane/32) + v%4, i.e.
// S[(32,4,2,4):(1@laneid,4@m,32@laneid,1@m)].
constexpr TileLayout mfma32x32_acc_swapped()
{
    TileLayout t;
    t.S(32, 1, laneid).S(4, 4, m).S(2, 32, laneid).S(4, 1, m);
    return t;
}

// Operand fragment of v_mfma_f32_16x16x32_f16 over a logical 16×32 (row, k)
// tile: lane = row + 16·(k / 8), register element = k mod 8, i.e.
// S[(16,4,8):(1@laneid,16@laneid,1@m)].
constexpr TileLayout mfma16x16x32_operand()
{
    TileLayout t;
    t.S(16, 1, laneid).S(4, 16, laneid).S(8, 1, m);
    return t;
}

// Accumulator of v_mfma_f32_16x16x32_f16 with the inputs swapped, over a
// logical 16×16 tile of D: D row = lane % 16, D col = 4·(lane/16) + v, i.e.
// S[(16,4,4):(1@laneid,16@laneid,1@m)].
constexpr TileLayout mfma16x16_acc_swapped()
{
    TileLayout t;
    t.S(16, 1, laneid).S(4, 16, laneid).S(4, 1, m);
    return t;
}

// ------------------------------------------------------------- checks

// The kernels' LDS chunk address fn(r, c) (element offset of 16-byte chunk c
// of row r) equals layout L for every element of a (rows × 64) tile.
template <class F>
constexpr bool check_swizzled_tile(const ComposeLayout &L, int rows, int cols, F fn)
{
    if (!L.well_formed())
        return false;
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols / 8; ++c)
            for (int e = 0; e < 8; ++e)
                if (fn(r, c) + e != L.apply2(r, c * 8 + e, cols))
                    return false;
    return true;
}

// A fragment read by lane l, element e, of chunk (K-step base) + hi(l) of row
// row(l) matches the operand layout L of a rows × kw MFMA slice for every
// (row, k): by default v_mfma_f32_32x32x16_f16's 32×16 slice.
template <class RowF, class HiF>
constexpr bool check_operand_fragment(RowF row_of_lane, HiF hi_of_lane,
                                      const TileLayout &L = mfma32x32x16_operand(), int kw = 16)
{
    for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
            const int64_t k = hi_of_lane(l) * 8 + e;
            const Coord c = L.apply2(row_of_lane(l), k, kw);
            if (c[laneid] != l || c[m] != e)
                return false;
        }
    return true;
}

// The epilogue's (lane, register) → (D row, D col) map equals the swapped
// accumulator layout L of an mf × mf MFMA tile (by default
// mfma32x32_acc_swapped), and is a bijection onto the tile.
template <class RowF, class ColF>
constexpr bool check_acc_fragment(RowF drow, ColF dcol, const TileLayout &L = mfma32x32_acc_swapped(),
                                  int mf = 32)
{
    bool seen[32 * 32] = {};
    for (int l = 0; l < 64; ++l)
        for (int v = 0; v < mf * mf / 64; ++v) {
            const int r = drow(l, v), c = dcol(l, v);
            if (r < 0 || r >= mf || c < 0 || c >= mf || seen[r * mf + c])
                return false;
            seen[r * mf + c] = true;
            const Coord x = L.apply2(r, c, mf);
            if (x[laneid] != l || x[m] != v)
                return false;
        }
    return true;
}

// ------------------------------------------------------- LDS bank model

// Cycles an LDS access takes under a simple bank model: lanes are served in
// passes of `lanes_per_pass`; within a pass each bank (bank_bytes wide,
// n_banks of them) serves one distinct word per cycle, so the pass costs the
// largest number of distinct words any bank sees.  `byte_addr[l]` is the
// first byte lane l accesses, `width` the bytes per lane (an access narrower
// than a bank touches one word).
constexpr int64_t lds_access_cycles(const int64_t *byte_addr, int lanes, int width, int n_banks,
                                    int bank_bytes, int lanes_per_pass)
{
    int64_t total = 0;
    for (int p0 = 0; p0 < lanes; p0 += lanes_per_pass) {
        int64_t worst = 0;
        for (int b = 0; b < n_banks; ++b) {
            // distinct words mapped to bank b in this pass
            int64_t words[256] = {};
            int nw = 0;
            for (int l = p0; l < p0 + lanes_per_pass && l < lanes; ++l)
                for (int off = 0; off < width; off += bank_bytes) {
                    const int64_t w = (byte_addr[l] + off) / bank_bytes;
                    if (w % n_banks != b)
                        continue;
                    bool dup = false;
                    for (int q = 0; q < nw; ++q)
                        dup = dup || words[q] == w;
                    if (!dup && nw < 256)
                        words[nw++] = w;
                }
            worst = nw > worst ? nw : worst;
        }
        total += worst;
    }
    return total;
}

}  // namespace layout
}  // namespace tg
