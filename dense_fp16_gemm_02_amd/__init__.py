"""Python binding of libtg_gemm.so — the MI355X (gfx950) fp16/bf16 GEMM D = A·Bᵀ.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``csrc/tg_gemm.hip``.  There is no fallback: if the library is
not built, importing the functions below raises.

    tg_gemm_f16(A, B, D, M, N, K, lda, ldb, ldd, stream) -> status
    tg_gemm_f16_plan(A, B, D, M, N, K, lda, ldb, ldd) -> (status, name, tiles)
    tg_gemm_bf16(...), tg_gemm_bf16_plan(...)   the same for bfloat16 data
    tg_status_string(status) -> str
    tg_device_info() -> (status, compute_units, max_clock_khz, arch)
    gemm(A, B, out=None, stream=None) -> D   (torch wrapper; fp16 or bf16)

Pointers may be given as torch tensors (their ``data_ptr()``) or integers;
``stream`` may be a ``torch.cuda.Stream``, an integer hipStream_t or None
(the null stream).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["TG_OK", "TG_ERR_INVALID_ARG", "TG_ERR_LAUNCH", "TG_ERR_DEVICE", "TG_ERR_TOO_LARGE",
           "TG_ERR_LAYOUT", "TG_MFMA_F16_16X16X32", "TG_MFMA_F16_32X32X16", "TG_MFMA_BF16_16X16X32",
           "TG_MFMA_MXF8_32X32X64", "tg_gemm_mxf8", "tg_gemm_mxf8_plan", "tg_gemm_mxf8_packed",
           "tg_gemm_mxf8_packed_plan", "tg_mx_packed_bytes", "tg_mx_pack_scales",
           "TG_MX_E4M3", "TG_MX_E5M2", "tg_gemm_mx", "tg_gemm_mx_plan", "tg_gemm_mx_packed",
           "tg_gemm_mx_packed_plan",
           "TgError", "lib_path", "load", "tg_gemm_f16", "tg_gemm_f16_plan", "tg_gemm_bf16",
           "tg_gemm_bf16_plan", "tg_status_string", "tg_device_info", "tg_mfma_ceiling", "tg_hbm_read_ceiling",
           "tg_gemm_f16_xcd_stamps", "gemm"]

TG_MX_E4M3 = 0  # block-scaled element encodings (include/tg_gemm.h)
TG_MX_E5M2 = 1
TG_OK = 0
TG_ERR_INVALID_ARG = -1
TG_ERR_LAUNCH = -2
TG_ERR_DEVICE = -3
TG_ERR_TOO_LARGE = -4
TG_ERR_LAYOUT = -5

# instruction codes of tg_mfma_ceiling (include/tg_ceiling.h)
TG_MFMA_F16_16X16X32 = 16
TG_MFMA_F16_32X32X16 = 32
TG_MFMA_BF16_16X16X32 = 17
TG_MFMA_MXF8_32X32X64 = 64

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtg_gemm.so")
_lib = None


class TgError(RuntimeError):
    def __init__(self, status: int, what: str = "tg_gemm_f16"):
        self.status = status
        super().__init__(f"{what} failed: {tg_status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libtg_gemm.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m dense_fp16_gemm_02_amd.build` "
            "(hipcc, gfx950) first")
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    for fn in (lib.tg_gemm_f16, lib.tg_gemm_bf16):
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    for fn in (lib.tg_gemm_f16_plan, lib.tg_gemm_bf16_plan):
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64,
                       ctypes.c_char_p, i64, ctypes.POINTER(i64)]
    lib.tg_gemm_mxf8.restype = ctypes.c_int
    lib.tg_gemm_mxf8.argtypes = [vp] * 5 + [i64] * 8 + [vp]
    lib.tg_gemm_mxf8_plan.restype = ctypes.c_int
    lib.tg_gemm_mxf8_plan.argtypes = [vp] * 5 + [i64] * 8 + [ctypes.c_char_p, i64, ctypes.POINTER(i64)]
    lib.tg_gemm_mxf8_packed.restype = ctypes.c_int
    lib.tg_gemm_mxf8_packed.argtypes = [vp] * 5 + [i64] * 6 + [vp]
    lib.tg_gemm_mxf8_packed_plan.restype = ctypes.c_int
    lib.tg_gemm_mxf8_packed_plan.argtypes = [vp] * 5 + [i64] * 6 + [ctypes.c_char_p, i64, ctypes.POINTER(i64)]
    ci = ctypes.c_int
    lib.tg_gemm_mx.restype = ctypes.c_int
    lib.tg_gemm_mx.argtypes = [vp] * 5 + [i64] * 8 + [ci, ci, vp]
    lib.tg_gemm_mx_plan.restype = ctypes.c_int
    lib.tg_gemm_mx_plan.argtypes = [vp] * 5 + [i64] * 8 + [ci, ci, ctypes.c_char_p, i64, ctypes.POINTER(i64)]
    lib.tg_gemm_mx_packed.restype = ctypes.c_int
    lib.tg_gemm_mx_packed.argtypes = [vp] * 5 + [i64] * 6 + [ci, ci, vp]
    lib.tg_gemm_mx_packed_plan.restype = ctypes.c_int
    lib.tg_gemm_mx_packed_plan.argtypes = [vp] * 5 + [i64] * 6 + [ci, ci, ctypes.c_char_p, i64,
                                                                    ctypes.POINTER(i64)]
    lib.tg_mx_packed_bytes.restype = i64
    lib.tg_mx_packed_bytes.argtypes = [i64, i64]
    lib.tg_mx_pack_scales.restype = ctypes.c_int
    lib.tg_mx_pack_scales.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.tg_status_string.restype = ctypes.c_char_p
    lib.tg_status_string.argtypes = [ctypes.c_int]
    lib.tg_mfma_ceiling.restype = ctypes.c_int
    lib.tg_mfma_ceiling.argtypes = [ctypes.c_int, vp, i64, vp, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, vp, vp]
    lib.tg_hbm_read_ceiling.restype = ctypes.c_int
    lib.tg_hbm_read_ceiling.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    lib.tg_gemm_f16_xcd_stamps.restype = ctypes.c_int
    lib.tg_gemm_f16_xcd_stamps.argtypes = [vp, vp, vp] + [i64] * 6 + [vp, i64, ctypes.POINTER(i64), vp]
    lib.tg_device_info.restype = ctypes.c_int
    lib.tg_device_info.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                   ctypes.c_char_p, i64]
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def tg_gemm_f16(A, B, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int, stream=None) -> int:
    """Enqueue D ← fp16_rne(A·Bᵀ) on ``stream``; returns the C status code."""
    return load().tg_gemm_f16(_ptr(A), _ptr(B), _ptr(D), M, N, K, lda, ldb, ldd, _stream(stream))


def tg_gemm_f16_plan(A, B, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int):
    """Host-only: (status, kernel name, output tile count) of the launch
    tg_gemm_f16 would make."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_f16_plan(_ptr(A), _ptr(B), _ptr(D), M, N, K, lda, ldb, ldd, buf, 128,
                                 ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_gemm_bf16(A, B, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int, stream=None) -> int:
    """Enqueue D ← bf16_rne(A·Bᵀ) on ``stream`` (bfloat16 data); returns the C status code."""
    return load().tg_gemm_bf16(_ptr(A), _ptr(B), _ptr(D), M, N, K, lda, ldb, ldd, _stream(stream))


def tg_gemm_bf16_plan(A, B, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int):
    """Host-only: (status, kernel name, output tile count) for tg_gemm_bf16."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_bf16_plan(_ptr(A), _ptr(B), _ptr(D), M, N, K, lda, ldb, ldd, buf, 128,
                                  ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_gemm_mxf8(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldsa: int, ldb: int, ldsb: int,
                 ldd: int, stream=None) -> int:
    """Enqueue the block-scaled FP8 GEMM (E4M3 bytes A, B; UE8M0 scale bytes
    SA, SB per 32 K; fp16 D) on ``stream``; returns the C status code."""
    return load().tg_gemm_mxf8(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldsa, ldb,
                               ldsb, ldd, _stream(stream))


def tg_gemm_mxf8_plan(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldsa: int, ldb: int, ldsb: int,
                      ldd: int):
    """Host-only: (status, kernel name, output tile count) for tg_gemm_mxf8."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_mxf8_plan(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldsa, ldb,
                                  ldsb, ldd, buf, 128, ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_gemm_mxf8_packed(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int,
                        stream=None) -> int:
    """Enqueue the block-scaled FP8 GEMM with SA and SB in the packed scale
    layout (include/tg_gemm.h); returns the C status code."""
    return load().tg_gemm_mxf8_packed(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldb, ldd,
                                      _stream(stream))


def tg_gemm_mxf8_packed_plan(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int):
    """Host-only: (status, kernel name, output tile count) for tg_gemm_mxf8_packed."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_mxf8_packed_plan(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldb, ldd,
                                         buf, 128, ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_gemm_mx(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldsa: int, ldb: int, ldsb: int,
               ldd: int, a_format: int, b_format: int, stream=None) -> int:
    """tg_gemm_mxf8 with the element encodings of A and B chosen separately
    (TG_MX_E4M3 or TG_MX_E5M2); returns the C status code."""
    return load().tg_gemm_mx(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldsa, ldb, ldsb,
                             ldd, a_format, b_format, _stream(stream))


def tg_gemm_mx_plan(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldsa: int, ldb: int, ldsb: int,
                    ldd: int, a_format: int, b_format: int):
    """Host-only: (status, kernel name, output tile count) for tg_gemm_mx."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_mx_plan(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldsa, ldb, ldsb,
                                ldd, a_format, b_format, buf, 128, ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_gemm_mx_packed(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int,
                      a_format: int, b_format: int, stream=None) -> int:
    """tg_gemm_mxf8_packed with the element encodings chosen separately."""
    return load().tg_gemm_mx_packed(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldb, ldd,
                                    a_format, b_format, _stream(stream))


def tg_gemm_mx_packed_plan(A, SA, B, SB, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int,
                           a_format: int, b_format: int):
    """Host-only: (status, kernel name, output tile count) for tg_gemm_mx_packed."""
    buf = ctypes.create_string_buffer(128)
    tiles = ctypes.c_int64(0)
    st = load().tg_gemm_mx_packed_plan(_ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(D), M, N, K, lda, ldb, ldd,
                                       a_format, b_format, buf, 128, ctypes.byref(tiles))
    return st, buf.value.decode(), tiles.value


def tg_mx_packed_bytes(rows: int, K: int) -> int:
    """Bytes of the packed scale layout for ``rows`` rows and K (-1: invalid)."""
    return load().tg_mx_packed_bytes(rows, K)


def tg_mx_pack_scales(S, rows: int, K: int, lds: int, P, stream=None) -> int:
    """Enqueue the row-major → packed scale conversion; returns the C status code."""
    return load().tg_mx_pack_scales(_ptr(S), rows, K, lds, _ptr(P), _stream(stream))


def tg_mfma_ceiling(shape: int, A, a_elems: int, B, b_elems: int, waves_per_simd: int, iters: int,
                    workgroups: int, out, stream=None) -> int:
    """Enqueue one launch of the matrix-core stream (measurement only; see
    include/tg_ceiling.h); returns the C status code."""
    return load().tg_mfma_ceiling(shape, _ptr(A), a_elems, _ptr(B), b_elems, waves_per_simd, iters,
                                  workgroups, _ptr(out), _stream(stream))


def tg_hbm_read_ceiling(src, nbytes: int, workgroups: int, out, stream=None) -> int:
    """Enqueue one streaming read of nbytes at src (measurement only; see
    include/tg_ceiling.h); returns the C status code."""
    return load().tg_hbm_read_ceiling(_ptr(src), nbytes, workgroups, _ptr(out), _stream(stream))


def tg_gemm_f16_xcd_stamps(A, B, D, M: int, N: int, K: int, lda: int, ldb: int, ldd: int, stamps,
                           stamps_len: int, stream=None):
    """tg_gemm_f16 through the stamping persistent kernel (measurement only;
    see include/tg_ceiling.h): (status, workgroups launched).  stamps: device
    buffer of stamps_len 64-bit words, three per workgroup."""
    wg = ctypes.c_int64(0)
    st = load().tg_gemm_f16_xcd_stamps(_ptr(A), _ptr(B), _ptr(D), M, N, K, lda, ldb, ldd, _ptr(stamps),
                                       stamps_len, ctypes.byref(wg), _stream(stream))
    return st, wg.value


def tg_status_string(status: int) -> str:
    return load().tg_status_string(status).decode()


def tg_device_info():
    """(status, compute_units, max_clock_khz, arch) of the current device."""
    cus, clk = ctypes.c_int(0), ctypes.c_int(0)
    arch = ctypes.create_string_buffer(64)
    st = load().tg_device_info(ctypes.byref(cus), ctypes.byref(clk), arch, len(arch))
    return st, cus.value, clk.value, arch.value.decode()


def gemm(A, B, out=None, stream=None):
    """torch convenience: D = A·Bᵀ for fp16 or bf16 GPU tensors A (M×K) and
    B (N×K) of the same dtype on one device, whose last dimension is
    contiguous and whose row stride is at least the row length (K for A and
    B, N for ``out``); D has that dtype.  Uses torch's current stream when
    ``stream`` is None.  Raises TypeError / ValueError on tensors the C ABI
    cannot take as they are (CPU tensors, mixed devices, overlapping rows such
    as a stride-0 ``expand``) and TgError on a non-zero status."""
    import torch

    if A.dtype != B.dtype or A.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("A and B must both be float16 or both bfloat16")
    if not A.is_cuda or not B.is_cuda or B.device != A.device:
        raise ValueError("A and B must be GPU tensors on the same device")
    dt = A.dtype
    call = tg_gemm_f16 if dt == torch.float16 else tg_gemm_bf16
    if A.dim() != 2 or B.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B must be 2-D with a contiguous last dimension")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"K mismatch: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=A.device)
    elif out.dtype != dt or out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be a {dt} (M, N) tensor with a contiguous last dimension")
    elif not out.is_cuda or out.device != A.device:
        raise ValueError("out must be on the device of A and B")
    # A row stride below the row length would make rows overlap (a stride-0
    # expand, for instance); the kernels read and write whole rows at the
    # given stride, so such views are refused rather than widened.  With one
    # row the stride is never used.
    for name, t, rows, width in (("A", A, M, K), ("B", B, N, K), ("out", out, M, N)):
        if rows > 1 and t.stride(0) < width:
            raise ValueError(f"{name} has row stride {t.stride(0)} < row length {width}; "
                             "pass a tensor with non-overlapping rows (e.g. .contiguous())")
    lda = A.stride(0) if M > 1 else max(K, 1)
    ldb = B.stride(0) if N > 1 else max(K, 1)
    ldd = out.stride(0) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    st = call(A, B, out, M, N, K, lda, ldb, ldd, stream)
    if st != TG_OK:
        raise TgError(st, call.__name__)
    return out
