"""Python view of the TileLayout helper in libtg_gemm.so (host-only calls).

    apply(spec, *coord, shape=None) -> {axis: value}   base coordinate D(x)+O
    replicas(spec) -> [{axis: value}, ...]             replica offsets r in R
    size(spec) -> int
    swizzle(per_element, swizzle_len, atom_len, addr, inner=True) -> int
    compose_apply(per_element, swizzle_len, atom_len, tile_spec, flat, inner=True) -> int
    lds_access_cycles(byte_addrs, width, n_banks, bank_bytes, lanes_per_pass) -> int

``spec`` uses the S[...] + R[...] + v@axis notation of the TIRx layout
pages (see include/tg_layout.h).
"""
from __future__ import annotations

import ctypes

from . import load as _load_core

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = _load_core()
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.tg_layout_num_axes.restype = ctypes.c_int
    lib.tg_layout_axis_name.restype = ctypes.c_char_p
    lib.tg_layout_axis_name.argtypes = [ctypes.c_int]
    lib.tg_layout_apply.restype = ctypes.c_int
    lib.tg_layout_apply.argtypes = [ctypes.c_char_p, vp, ctypes.c_int, vp, ctypes.c_int, vp,
                                    ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
    lib.tg_layout_size.restype = i64
    lib.tg_layout_size.argtypes = [ctypes.c_char_p]
    lib.tg_layout_replica_count.restype = i64
    lib.tg_layout_replica_count.argtypes = [ctypes.c_char_p]
    lib.tg_layout_replica.restype = ctypes.c_int
    lib.tg_layout_replica.argtypes = [ctypes.c_char_p, i64, vp, ctypes.c_int]
    lib.tg_swizzle.restype = i64
    lib.tg_swizzle.argtypes = [ctypes.c_int] * 4 + [i64]
    lib.tg_compose_apply.restype = i64
    lib.tg_compose_apply.argtypes = [ctypes.c_int] * 4 + [ctypes.c_char_p, i64]
    lib.tg_lds_access_cycles.restype = i64
    lib.tg_lds_access_cycles.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


class LayoutError(ValueError):
    pass


def axis_names():
    lib = _load()
    return [lib.tg_layout_axis_name(i).decode() for i in range(lib.tg_layout_num_axes())]


def _coord_dict(vals, mask=None, keep_zero=False):
    names = axis_names()
    out = {}
    for i, n in enumerate(names):
        used = mask is not None and (mask >> i) & 1
        if used or (keep_zero and vals[i]) or (mask is None and vals[i]):
            out[n] = int(vals[i])
    return out


def apply(spec: str, *coord: int, shape=None) -> dict:
    """Base coordinate of one element (replicas are not enumerated).  With
    ``shape`` the coordinate is a logical one flattened row-major; otherwise
    one integer is a flat index and several are shard components."""
    lib = _load()
    n = lib.tg_layout_num_axes()
    c = (ctypes.c_int64 * len(coord))(*coord)
    out = (ctypes.c_int64 * n)()
    used = ctypes.c_uint32(0)
    if shape is not None:
        shp = (ctypes.c_int64 * len(shape))(*shape)
        rc = lib.tg_layout_apply(spec.encode(), c, len(coord), shp, len(shape), out, n,
                                 ctypes.byref(used))
    else:
        rc = lib.tg_layout_apply(spec.encode(), c, len(coord), None, 0, out, n,
                                 ctypes.byref(used))
    if rc != 0:
        raise LayoutError(f"apply({spec!r}, {coord}, shape={shape}) failed ({rc})")
    return _coord_dict(list(out), used.value)


def size(spec: str) -> int:
    v = _load().tg_layout_size(spec.encode())
    if v < 0:
        raise LayoutError(f"cannot parse {spec!r}")
    return int(v)


def replicas(spec: str) -> list:
    lib = _load()
    cnt = lib.tg_layout_replica_count(spec.encode())
    if cnt < 0:
        raise LayoutError(f"cannot parse {spec!r}")
    n = lib.tg_layout_num_axes()
    res = []
    for r in range(cnt):
        out = (ctypes.c_int64 * n)()
        if lib.tg_layout_replica(spec.encode(), r, out, n) != 0:
            raise LayoutError(f"replica {r} of {spec!r}")
        res.append(_coord_dict(list(out)))
    return res


def swizzle(per_element: int, swizzle_len: int, atom_len: int, addr: int, inner: bool = True) -> int:
    v = _load().tg_swizzle(per_element, swizzle_len, atom_len, int(inner), addr)
    if v < 0:
        raise LayoutError("invalid swizzle parameters or address")
    return int(v)


def compose_apply(per_element: int, swizzle_len: int, atom_len: int, tile_spec: str, flat: int,
                  inner: bool = True) -> int:
    v = _load().tg_compose_apply(per_element, swizzle_len, atom_len, int(inner),
                                 tile_spec.encode(), flat)
    if v < 0:
        raise LayoutError(f"compose_apply failed ({v})")
    return int(v)


def lds_access_cycles(byte_addrs, width: int, n_banks: int, bank_bytes: int,
                      lanes_per_pass: int) -> int:
    arr = (ctypes.c_int64 * len(byte_addrs))(*[int(a) for a in byte_addrs])
    v = _load().tg_lds_access_cycles(arr, len(byte_addrs), width, n_banks, bank_bytes,
                                     lanes_per_pass)
    if v < 0:
        raise LayoutError("invalid bank-model arguments")
    return int(v)
