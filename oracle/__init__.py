"""CPU oracle for the fp16 (and bf16, and block-scaled FP8) GEMM D = A·Bᵀ —
test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The GPU library never does,
and this package never imports the GPU library: the two share no code.

The arithmetic lives in ``gemm_oracle.c`` (plain C, fp64 accumulation, direct
fp64→fp16 round-to-nearest-even); this module builds it with gcc, loads it
with ctypes and adds the acceptance check used by the parity tests.

Acceptance (per checked element): |D − ref| ≤ 4e-3·bound + ulp16(ref) and D
finite, where bound = Σ_k |A_ik|·|B_jk| and ulp16(x) is the spacing of
binary16 at |x|: 2^(⌊log2|x|⌋−10) for |x| ≥ 2^−14, else 2^−24.  For bfloat16
the output term is ulp_bf16(ref) = 2^(⌊log2|x|⌋−7) (2^−133 below 2^−126).

bfloat16 arrays are passed and returned as uint16 bit patterns (numpy has no
bfloat16 type); ``fmt="bf16"`` selects that format everywhere.

``gemm_mx`` is the block-scaled FP8 GEMM: E4M3 operand bytes, one UE8M0 scale
byte per 32 K elements of each row, fp16 output; its bound is
Σ_k |sa·a|·|sb·b| and the acceptance check is the fp16 one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "libgemm_oracle.so")

REL_TOL = 4e-3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libgemm_oracle.so``."""
    global _lib
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_double_to_half.restype = ctypes.c_uint16
    lib.oracle_double_to_half.argtypes = [ctypes.c_double]
    lib.oracle_half_to_double_array.restype = None
    lib.oracle_half_to_double_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_double_to_half_array.restype = None
    lib.oracle_double_to_half_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_bf16_to_double_array.restype = None
    lib.oracle_bf16_to_double_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_double_to_bf16_array.restype = None
    lib.oracle_double_to_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_e4m3_to_double_array.restype = None
    lib.oracle_e4m3_to_double_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_e8m0_to_double.restype = ctypes.c_double
    lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e5m2_to_double_array.restype = None
    lib.oracle_e5m2_to_double_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_gemm_mxf8.restype = ctypes.c_int
    lib.oracle_gemm_mxf8.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 7 + [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    lib.oracle_gemm_mx.restype = ctypes.c_int
    lib.oracle_gemm_mx.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 7 + [ctypes.c_int] * 2 + [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    for fn in (lib.oracle_gemm_f16, lib.oracle_gemm_bf16):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def half_to_double(h: np.ndarray) -> np.ndarray:
    """Exact binary16 → float64 decode (oracle's own bit decode)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_half_to_double_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


def double_to_half_bits(x: np.ndarray) -> np.ndarray:
    """float64 → binary16 bits, round-to-nearest-even from float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_double_to_half_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_double(h: np.ndarray) -> np.ndarray:
    """Exact bfloat16 (uint16 bits) → float64 decode."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_bf16_to_double_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


def double_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 → bfloat16 bits, round-to-nearest-even from float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_double_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e4m3_to_double(b: np.ndarray) -> np.ndarray:
    """Exact FP8 E4M3 (uint8 codes) → float64 decode (NaN for 0x7f, 0xff)."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_e4m3_to_double_array(b.ctypes.data, out.ctypes.data, b.size)
    return out


def e5m2_to_double(b: np.ndarray) -> np.ndarray:
    """Exact FP8 E5M2 (uint8 codes) → float64 decode (±inf for 0x7c, 0xfc;
    NaN for the other codes with all exponent bits set)."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_e5m2_to_double_array(b.ctypes.data, out.ctypes.data, b.size)
    return out


MX_FORMATS = {"e4m3": 0, "e5m2": 1}


def e8m0_to_double(s: np.ndarray) -> np.ndarray:
    """UE8M0 scale bytes → float64 powers of two (NaN for 255)."""
    s = np.asarray(s, dtype=np.uint8)
    f = _load().oracle_e8m0_to_double
    return np.vectorize(lambda v: f(int(v)), otypes=[np.float64])(s) if s.size else np.zeros(s.shape)


def decode(x: np.ndarray, fmt: str) -> np.ndarray:
    """float64 values of fp16 data (fmt "f16") or bf16 bit patterns ("bf16")."""
    if fmt == "bf16":
        return bf16_to_double(x)
    return np.asarray(x, dtype=np.float16).astype(np.float64)


class Result:
    """Oracle output for the requested rows: fp16 D, fp64 bound and fp64 sum."""

    def __init__(self, d: np.ndarray, bound: np.ndarray, total: np.ndarray, rows: np.ndarray,
                 fmt: str = "f16"):
        self.d = d          # float16 values, or uint16 bf16 bit patterns
        self.bound = bound
        self.sum = total
        self.rows = rows
        self.fmt = fmt


def gemm(a: np.ndarray, b: np.ndarray, M: int, N: int, K: int,
         rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
         fmt: str = "f16") -> Result:
    """Reference D = A·Bᵀ on fp16 arrays ``a`` (M×lda) and ``b`` (N×ldb), or
    on bf16 bit arrays with ``fmt="bf16"``.

    Returns the requested rows (all rows if ``rows`` is None) as a dense
    (len(rows), N) float16 array (uint16 bf16 bits for bf16), with bound and
    the fp64 sum beside it.
    """
    if fmt not in ("f16", "bf16"):
        raise ValueError("fmt must be 'f16' or 'bf16'")
    et = np.uint16 if fmt == "bf16" else np.float16
    a = np.ascontiguousarray(a, dtype=et)
    b = np.ascontiguousarray(b, dtype=et)
    if a.ndim != 2 or b.ndim != 2 or a.shape[0] < M or b.shape[0] < N:
        raise ValueError("operand shapes do not cover M/N")
    lda, ldb = a.shape[1], b.shape[1]
    if M == 0:
        lda = max(lda, K)
    if N == 0:
        ldb = max(ldb, K)
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    d = np.zeros((nrows, N), dtype=et)
    bound = np.zeros((nrows, N), dtype=np.float64)
    total = np.zeros((nrows, N), dtype=np.float64)
    nt = default_threads() if nthreads is None else nthreads
    fn = _load().oracle_gemm_bf16 if fmt == "bf16" else _load().oracle_gemm_f16
    rc = fn(
        a.ctypes.data if a.size else None, b.ctypes.data if b.size else None,
        d.ctypes.data if d.size else None, bound.ctypes.data if bound.size else None,
        total.ctypes.data if total.size else None,
        M, N, K, lda, ldb,
        rows_arr.ctypes.data if rows_arr is not None and rows_arr.size else None,
        nrows, nt)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out_rows = np.arange(M, dtype=np.int64) if rows is None else rows_arr
    return Result(d, bound, total, out_rows, fmt)


def gemm_mx(a: np.ndarray, sa: np.ndarray, b: np.ndarray, sb: np.ndarray, M: int, N: int, K: int,
            rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None,
            a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> Result:
    """Reference block-scaled FP8 GEMM on uint8 arrays: ``a`` (M×lda FP8
    codes in the encoding ``a_fmt``, "e4m3" or "e5m2"), ``sa`` (M×ldsa UE8M0
    scale bytes, one per 32 K elements), and likewise ``b``, ``sb`` for the N
    rows of B.  Returns fp16 D for the requested rows with the float64 sum
    and bound beside it."""
    if a_fmt not in MX_FORMATS or b_fmt not in MX_FORMATS:
        raise ValueError("element encodings are 'e4m3' or 'e5m2'")
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    if min(a.ndim, b.ndim, sa.ndim, sb.ndim) != 2 or a.shape[0] < M or b.shape[0] < N or \
            sa.shape[0] < M or sb.shape[0] < N:
        raise ValueError("operand shapes do not cover M/N")
    blocks = (K + 31) // 32
    lda, ldb = max(a.shape[1], K if M == 0 else 0), max(b.shape[1], K if N == 0 else 0)
    ldsa, ldsb = max(sa.shape[1], blocks if M == 0 else 0), max(sb.shape[1], blocks if N == 0 else 0)
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    d = np.zeros((nrows, N), dtype=np.float16)
    bound = np.zeros((nrows, N), dtype=np.float64)
    total = np.zeros((nrows, N), dtype=np.float64)
    nt = default_threads() if nthreads is None else nthreads
    ptr = lambda x: x.ctypes.data if x.size else None
    rc = _load().oracle_gemm_mx(
        ptr(a), ptr(sa), ptr(b), ptr(sb), ptr(d), ptr(bound), ptr(total),
        M, N, K, lda, ldsa, ldb, ldsb, MX_FORMATS[a_fmt], MX_FORMATS[b_fmt],
        rows_arr.ctypes.data if rows_arr is not None and rows_arr.size else None, nrows, nt)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out_rows = np.arange(M, dtype=np.int64) if rows is None else rows_arr
    return Result(d, bound, total, out_rows, "f16")


def ulp16(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 at |x| (2^-24 in the subnormal range and at 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(ax.shape, 2.0 ** -24)
    big = ax >= 2.0 ** -14
    if np.any(big):
        e = np.floor(np.log2(ax[big]))
        out[big] = np.exp2(e - 10)
    return out


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 at |x| (2^-133 in the subnormal range and at 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(ax.shape, 2.0 ** -133)
    big = ax >= 2.0 ** -126
    if np.any(big):
        e = np.floor(np.log2(ax[big]))
        out[big] = np.exp2(e - 7)
    return out


def tolerance(ref: np.ndarray, bound: np.ndarray, fmt: str = "f16") -> np.ndarray:
    if fmt == "bf16":
        return REL_TOL * bound + ulp_bf16(bf16_to_double(ref))
    return REL_TOL * bound + ulp16(ref.astype(np.float64))


def check(d_gpu: np.ndarray, res: Result, cols: Optional[np.ndarray] = None):
    """Apply the acceptance inequality to every element of ``d_gpu`` (shape
    (len(res.rows), N) or restricted to ``cols``).  Returns (ok, worst_ratio,
    report) where worst_ratio = max |D−ref| / tol (≤ 1 passes)."""
    ref = res.d if cols is None else res.d[:, cols]
    bound = res.bound if cols is None else res.bound[:, cols]
    d = np.asarray(d_gpu, dtype=np.uint16 if res.fmt == "bf16" else np.float16)
    if d.shape != ref.shape:
        raise ValueError(f"shape mismatch {d.shape} vs {ref.shape}")
    if d.size == 0:
        return True, 0.0, "empty"
    dd = decode(d, res.fmt)
    rr = decode(ref, res.fmt)
    finite = np.isfinite(dd)
    tol = tolerance(ref, bound, res.fmt)
    err = np.abs(dd - rr)
    err = np.where(finite, err, np.inf)
    ratio = err / tol
    worst = float(np.max(ratio))
    ok = bool(np.all(finite)) and worst <= 1.0
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    report = (f"worst err/tol={worst:.4g} at (row {int(res.rows[idx[0]])}, col {idx[1]}): "
              f"gpu={dd[idx]!r} ref={rr[idx]!r} tol={tol[idx]:.4g}; "
              f"non-finite={int(np.size(d) - np.count_nonzero(finite))}")
    return ok, worst, report
