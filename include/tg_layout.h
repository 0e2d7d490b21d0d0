/*
 * tg_layout.h — host-only C ABI of the TileLayout helper in libtg_gemm.so.
 * None of these calls touches a GPU.
 *
 * Layout notation ("TIRx Layout API", sections "TileLayout", "Shard",
 * "Replica", "Offset", "组合三个部分"):
 *
 *     S[(e0, e1, ...):(s0@a0, s1@a1, ...)] + R[(r0, ...):(t0@b0, ...)] + v@axis
 *
 * A bare integer extent and stride may stand for a 1-tuple; a stride with no
 * "@axis" goes to the default linear axis m.  Axis names: m, laneid, warpid,
 * tx, wgid, tid_in_wg, wid_in_wg, bx, by, bz, cbx, cby, cbz, TLane, TCol.
 * L(x) = { D(x) + r + O | r in R }: D(x) splits the row-major flat index by
 * the shard extents and adds c_k·s_k to axis a_k ("正向映射").
 *
 * Every function returns a negative value on a parse error or an argument
 * out of range; it writes outputs only on success.
 */
#ifndef TG_LAYOUT_H
#define TG_LAYOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of named axes; an axis id is an index in [0, tg_layout_num_axes()). */
int tg_layout_num_axes(void);
/* Static name of axis `id`, or "?" when out of range. */
const char *tg_layout_axis_name(int id);

/*
 * tg_layout_apply — base coordinate D(x) + O of one logical element; replicas
 * are not enumerated ("正向映射").  The three input forms:
 *   shape == NULL, ncoord == 1          → apply(linear_coord)
 *   shape == NULL, ncoord == #shard     → apply(*shard_coord)
 *   shape != NULL, nshape == ncoord     → apply(*logical_coord, shape=shape)
 * The flat index must lie below the product of the shard extents.
 * out[0..out_len) receives the value on every axis (out_len >= number of
 * axes); *used (may be NULL) receives a bit mask of the axes the shard or the
 * offset touches.  Returns 0 or a negative error.
 */
int tg_layout_apply(const char *spec, const int64_t *coord, int ncoord, const int64_t *shape,
                    int nshape, int64_t *out, int out_len, uint32_t *used);

/* Number of logical elements the shard covers, or a negative error. */
int64_t tg_layout_size(const char *spec);

/* Number of replica offsets (1 when there is no R[...]), or a negative error. */
int64_t tg_layout_replica_count(const char *spec);

/* The r-th replica offset (row-major over the replica extents) into
 * out[0..out_len).  Returns 0 or a negative error. */
int tg_layout_replica(const char *spec, int64_t r, int64_t *out, int out_len);

/*
 * tg_swizzle — XOR swizzle of a linear element address ("Swizzle 变换"):
 * keep the low `per_element` bits; of the rest, x, XOR bits
 * [atom_len, atom_len+swizzle_len) into bits [0, swizzle_len) when `inner` is
 * nonzero, or bits [0, swizzle_len) into [atom_len, atom_len+swizzle_len)
 * otherwise.  Returns the swizzled address, or -1 unless
 * atom_len >= swizzle_len >= 0, per_element >= 0 and addr >= 0.
 */
int64_t tg_swizzle(int per_element, int swizzle_len, int atom_len, int inner, int64_t addr);

/*
 * tg_compose_apply — ComposeLayout(per_element, swizzle_len, atom_len,
 * tile_layout=tile_spec, swizzle_inner=inner) at flat logical index `flat`:
 * the tile's m coordinate, then the swizzle.  The tile may only produce the
 * m axis.  Returns the address or a negative error.
 */
int64_t tg_compose_apply(int per_element, int swizzle_len, int atom_len, int inner,
                         const char *tile_spec, int64_t flat);

/*
 * tg_lds_access_cycles — cycles one LDS access instruction takes under a
 * bank model: lanes are served `lanes_per_pass` at a time; in a pass each of
 * `n_banks` banks (`bank_bytes` wide) serves one distinct word per cycle.
 * byte_addr[l] is lane l's first byte and `width` its access size.
 * Returns the cycle count or a negative error.
 */
int64_t tg_lds_access_cycles(const int64_t *byte_addr, int lanes, int width, int n_banks,
                             int bank_bytes, int lanes_per_pass);

#ifdef __cplusplus
}
#endif

#endif /* TG_LAYOUT_H */
