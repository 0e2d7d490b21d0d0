// tile_layout_abi.cpp — parser for the S[...] + R[...] + offset notation and
// the host-only C ABI declared in include/tg_layout.h.
#include <stdint.h>
#include <string.h>

#include "tg_layout.h"
#include "tile_layout.hpp"

namespace {

using tg::layout::ComposeLayout;
using tg::layout::Coord;
using tg::layout::Iter;
using tg::layout::MAX_ITERS;
using tg::layout::NUM_AXES;
using tg::layout::Swizzle;
using tg::layout::TileLayout;

struct Parser {
    const char *s;
    bool ok = true;

    void ws()
    {
        while (*s == ' ' || *s == '\t' || *s == '\n' || *s == '\r')
            ++s;
    }
    bool eat(char c)
    {
        ws();
        if (*s == c) {
            ++s;
            return true;
        }
        return false;
    }
    void expect(char c)
    {
        if (!eat(c))
            ok = false;
    }
    bool integer(int64_t &v)
    {
        ws();
        bool neg = false;
        if (*s == '-' || *s == '+') {
            neg = *s == '-';
            ++s;
            ws();
        }
        if (*s < '0' || *s > '9')
            return false;
        int64_t x = 0;
        while (*s >= '0' && *s <= '9') {
            if (x > (INT64_MAX - 9) / 10) {
                ok = false;
                return false;
            }
            x = x * 10 + (*s - '0');
            ++s;
        }
        v = neg ? -x : x;
        return true;
    }
    int axis()
    {
        ws();
        const char *b = s;
        while ((*s >= 'a' && *s <= 'z') || (*s >= 'A' && *s <= 'Z') || (*s >= '0' && *s <= '9') ||
               *s == '_')
            ++s;
        const size_t n = (size_t)(s - b);
        for (int a = 0; a < NUM_AXES; ++a) {
            const char *nm = tg::layout::axis_name(a);
            if (strlen(nm) == n && strncmp(nm, b, n) == 0)
                return a;
        }
        ok = false;
        return -1;
    }
    // "v" or "v@axis"
    void stride(int64_t &v, int &ax)
    {
        if (!integer(v)) {
            ok = false;
            return;
        }
        ax = tg::layout::m;
        if (eat('@'))
            ax = axis();
    }
    // "(e0, e1, ...)" or "e"
    int extents(int64_t *e)
    {
        int n = 0;
        if (eat('(')) {
            do {
                if (n >= MAX_ITERS || !integer(e[n])) {
                    ok = false;
                    return 0;
                }
                ++n;
            } while (eat(','));
            expect(')');
        } else {
            if (!integer(e[0])) {
                ok = false;
                return 0;
            }
            n = 1;
        }
        return n;
    }
    int strides(int64_t *v, int *ax)
    {
        int n = 0;
        if (eat('(')) {
            do {
                if (n >= MAX_ITERS) {
                    ok = false;
                    return 0;
                }
                stride(v[n], ax[n]);
                ++n;
            } while (ok && eat(','));
            expect(')');
        } else {
            stride(v[0], ax[0]);
            n = 1;
        }
        return n;
    }
    // "[ extents : strides ]" appended to `it`
    int spec(Iter *it)
    {
        expect('[');
        int64_t e[MAX_ITERS] = {}, v[MAX_ITERS] = {};
        int ax[MAX_ITERS] = {};
        const int ne = extents(e);
        expect(':');
        const int nv = strides(v, ax);
        expect(']');
        if (!ok || ne != nv)
            return ok = false, 0;
        for (int k = 0; k < ne; ++k) {
            if (e[k] <= 0)
                return ok = false, 0;
            it[k] = Iter{e[k], v[k], ax[k]};
        }
        return ne;
    }
};

bool parse(const char *text, TileLayout &out)
{
    if (!text)
        return false;
    Parser p{text};
    TileLayout L;
    bool have_shard = false;
    do {
        p.ws();
        if (*p.s == 'S' && (p.s[1] == '[' || p.s[1] == ' ')) {
            ++p.s;
            if (have_shard)
                return false;
            L.n_shard = p.spec(L.shard);
            have_shard = true;
        } else if (*p.s == 'R' && (p.s[1] == '[' || p.s[1] == ' ')) {
            ++p.s;
            Iter it[MAX_ITERS];
            const int n = p.spec(it);
            for (int k = 0; k < n && p.ok; ++k) {
                if (L.n_replica >= MAX_ITERS)
                    return false;
                L.replica[L.n_replica++] = it[k];
            }
        } else {
            int64_t v = 0;
            int ax = 0;
            p.stride(v, ax);
            if (p.ok)
                L.offset[ax] += v;
        }
        if (!p.ok)
            return false;
    } while (p.eat('+'));
    p.ws();
    if (*p.s != 0 || !have_shard || L.n_shard == 0)
        return false;
    out = L;
    return true;
}

void write_coord(const Coord &c, int64_t *out)
{
    for (int a = 0; a < NUM_AXES; ++a)
        out[a] = c[a];
}

}  // namespace

extern "C" int tg_layout_num_axes(void) { return NUM_AXES; }

extern "C" const char *tg_layout_axis_name(int id) { return tg::layout::axis_name(id); }

extern "C" int tg_layout_apply(const char *spec, const int64_t *coord, int ncoord,
                               const int64_t *shape, int nshape, int64_t *out, int out_len,
                               uint32_t *used)
{
    TileLayout L;
    if (!parse(spec, L) || !out || out_len < NUM_AXES || !coord || ncoord <= 0)
        return -1;
    const int64_t size = L.size();
    Coord c;
    if (shape) {
        if (nshape != ncoord || ncoord > 16)
            return -2;
        int64_t flat = 0;
        for (int d = 0; d < ncoord; ++d) {
            if (shape[d] <= 0 || coord[d] < 0 || coord[d] >= shape[d])
                return -2;
            flat = flat * shape[d] + coord[d];
        }
        if (flat >= size)
            return -3;
        c = L.apply(coord, shape, ncoord);
    } else if (ncoord == 1) {
        if (coord[0] < 0 || coord[0] >= size)
            return -3;
        c = L.apply(coord[0]);
    } else if (ncoord == L.n_shard) {
        for (int k = 0; k < ncoord; ++k)
            if (coord[k] < 0 || coord[k] >= L.shard[k].extent)
                return -3;
        c = L.apply_shard(coord);
    } else {
        return -2;
    }
    write_coord(c, out);
    if (used) {
        uint32_t mask = 0;
        for (int a = 0; a < NUM_AXES; ++a)
            if (L.uses_axis(a))
                mask |= 1u << a;
        *used = mask;
    }
    return 0;
}

extern "C" int64_t tg_layout_size(const char *spec)
{
    TileLayout L;
    if (!parse(spec, L))
        return -1;
    return L.size();
}

extern "C" int64_t tg_layout_replica_count(const char *spec)
{
    TileLayout L;
    if (!parse(spec, L))
        return -1;
    return L.replica_count();
}

extern "C" int tg_layout_replica(const char *spec, int64_t r, int64_t *out, int out_len)
{
    TileLayout L;
    if (!parse(spec, L) || !out || out_len < NUM_AXES)
        return -1;
    if (r < 0 || r >= L.replica_count())
        return -3;
    write_coord(L.replica_offset(r), out);
    return 0;
}

extern "C" int64_t tg_swizzle(int per_element, int swizzle_len, int atom_len, int inner,
                              int64_t addr)
{
    const Swizzle sw{per_element, swizzle_len, atom_len, inner != 0};
    if (!sw.valid() || swizzle_len < 0 || per_element > 32 || atom_len + swizzle_len > 32 ||
        addr < 0)
        return -1;
    return sw(addr);
}

extern "C" int64_t tg_compose_apply(int per_element, int swizzle_len, int atom_len, int inner,
                                    const char *tile_spec, int64_t flat)
{
    ComposeLayout C;
    C.sw = Swizzle{per_element, swizzle_len, atom_len, inner != 0};
    if (!parse(tile_spec, C.tile) || swizzle_len < 0 || per_element > 32 ||
        atom_len + swizzle_len > 32)
        return -1;
    if (!C.well_formed())
        return -2;
    if (flat < 0 || flat >= C.tile.size())
        return -3;
    return C.apply(flat);
}

extern "C" int64_t tg_lds_access_cycles(const int64_t *byte_addr, int lanes, int width,
                                        int n_banks, int bank_bytes, int lanes_per_pass)
{
    if (!byte_addr || lanes <= 0 || lanes > 1024 || width <= 0 || n_banks <= 0 ||
        bank_bytes <= 0 || lanes_per_pass <= 0 || (width > bank_bytes && width % bank_bytes != 0) ||
        lanes_per_pass * ((width + bank_bytes - 1) / bank_bytes) > 256)
        return -1;
    for (int l = 0; l < lanes; ++l)
        if (byte_addr[l] < 0)
            return -1;
    return tg::layout::lds_access_cycles(byte_addr, lanes, width, n_banks, bank_bytes,
                                         lanes_per_pass);
}
