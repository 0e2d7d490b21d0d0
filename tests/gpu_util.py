"""Helpers for the GPU tests: move seeded numpy operands onto cuda:0, call
tg_gemm_f16 through the C ABI on a torch stream, and read back D together
with a guard band around its window."""
from __future__ import annotations

import sys

import numpy as np

SENTINEL = 0x7777  # a finite fp16 bit pattern (30576.0) no kernel output takes here


def say(msg: str) -> None:
    """Name the case before each GPU step (and flush) so a fault is attributable."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


NAN_BITS = {"f16": 0x7e00, "bf16": 0x7fc0}


def to_dev(x: np.ndarray, offset_elems: int = 0, fmt: str = "f16"):
    """Copy a 2-D 16-bit array (fp16 values, or bf16 bit patterns as uint16)
    into a device buffer starting `offset_elems` elements past a 256-byte
    aligned allocation (offset 1 misaligns it); the rest of the buffer holds
    NaN of that format."""
    import torch

    raw = np.ascontiguousarray(x).reshape(-1).view(np.uint16).view(np.int16)
    buf = torch.full((raw.size + offset_elems + 8,), NAN_BITS[fmt], dtype=torch.int16,
                     device="cuda:0")
    if raw.size:
        buf[offset_elems:offset_elems + raw.size].copy_(torch.from_numpy(raw))
    return buf, buf.data_ptr() + 2 * offset_elems


def run(a: np.ndarray, b: np.ndarray, M: int, N: int, K: int, *, ldd: int | None = None,
        guard: int = 0, a_off: int = 0, b_off: int = 0, d_off: int = 0, stream=None,
        label: str = "", fmt: str = "f16"):
    """D = A·Bᵀ on the GPU.  a is (M, lda) and b is (N, ldb) fp16, or bf16 bit
    patterns (uint16) with fmt="bf16" (padding columns beyond K are passed
    through untouched).  D lives in a buffer of (M + 2·guard) rows ×
    ldd_total columns filled with SENTINEL, with the window at (guard,
    guard).  Returns (D window as fp16 (M, N) — uint16 bits for bf16 — full
    buffer as uint16 for guard checks, status)."""
    import torch

    import dense_fp16_gemm_02_amd as tg

    lda = a.shape[1] if a.ndim == 2 and a.shape[1] else max(K, 1)
    ldb = b.shape[1] if b.ndim == 2 and b.shape[1] else max(K, 1)
    ldd = (N + 2 * guard) if ldd is None else ldd
    rows_total = M + 2 * guard
    a_buf, a_ptr = to_dev(a, a_off, fmt)
    b_buf, b_ptr = to_dev(b, b_off, fmt)
    d_buf = torch.full((rows_total * ldd + d_off + 8,), 0, dtype=torch.int16, device="cuda:0")
    d_buf.fill_(SENTINEL)
    d_ptr = d_buf.data_ptr() + 2 * (d_off + guard * ldd + guard)
    s = stream if stream is not None else torch.cuda.current_stream()
    say(f"{label} {fmt} M={M} N={N} K={K} lda={lda} ldb={ldb} ldd={ldd} guard={guard} "
        f"offs=({a_off},{b_off},{d_off})")
    call = tg.tg_gemm_bf16 if fmt == "bf16" else tg.tg_gemm_f16
    st = call(a_ptr, b_ptr, d_ptr, M, N, K, lda, ldb, ldd, s)
    s.synchronize()
    torch.cuda.synchronize()
    full = d_buf.cpu().numpy().view(np.uint16)[d_off:d_off + rows_total * ldd].reshape(rows_total, ldd)
    win = full[guard:guard + M, guard:guard + N]
    if fmt != "bf16":
        win = win.view(np.float16)
    del a_buf, b_buf
    return np.array(win), full, st


def guard_intact(full: np.ndarray, M: int, N: int, guard: int) -> bool:
    mask = np.ones(full.shape, dtype=bool)
    mask[guard:guard + M, guard:guard + N] = False
    return bool(np.all(full[mask] == SENTINEL))


def _bytes(x: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda:0")


def pack_scales(S, rows, K, lds):
    """The packed scale layout of a device buffer of row-major scales (rows ×
    lds bytes), made on the device by tg_mx_pack_scales."""
    import torch

    import dense_fp16_gemm_02_amd as tg

    nbytes = tg.tg_mx_packed_bytes(rows, K)
    assert nbytes >= 0
    P = torch.full((max(nbytes, 16),), 0xA5, dtype=torch.uint8, device="cuda:0")
    st = tg.tg_mx_pack_scales(S, rows, K, lds, P, torch.cuda.current_stream())
    assert st == tg.TG_OK, st
    return P


def run_mx(a, sa, b, sb, M, N, K, guard=0, label="", packed=False, a_fmt=0, b_fmt=0):
    """D (M, N) fp16 window and the full (M+2g, N+2g) buffer (uint16) of
    tg_gemm_mxf8 on byte arrays a (M, lda), sa (M, ldsa), b (N, ldb), sb
    (N, ldsb); every byte in them is passed to the device as is.  With
    packed=True the scales are first converted on the device into the packed
    layout (tg_mx_pack_scales) and tg_gemm_mxf8_packed runs instead.  Element
    encodings other than E4M3 on both operands (a_fmt, b_fmt: 0 E4M3, 1 E5M2)
    go through tg_gemm_mx / tg_gemm_mx_packed."""
    import torch

    import dense_fp16_gemm_02_amd as tg

    lda, ldsa, ldb, ldsb = a.shape[1], sa.shape[1], b.shape[1], sb.shape[1]
    ldd = N + 2 * guard
    A, SA, B, SB = _bytes(a), _bytes(sa), _bytes(b), _bytes(sb)
    d = torch.full(((M + 2 * guard) * ldd + 8,), SENTINEL, dtype=torch.int16, device="cuda:0")
    dptr = d.data_ptr() + 2 * (guard * ldd + guard)
    say(f"mxf8 {label} M={M} N={N} K={K} lda={lda} ldsa={ldsa} ldb={ldb} ldsb={ldsb} guard={guard} "
        f"packed={packed} formats=({a_fmt},{b_fmt})")
    s = torch.cuda.current_stream()
    if packed:
        PA, PB = pack_scales(SA, M, K, ldsa), pack_scales(SB, N, K, ldsb)
        if a_fmt or b_fmt:
            st = tg.tg_gemm_mx_packed(A, PA, B, PB, dptr, M, N, K, lda, ldb, ldd, a_fmt, b_fmt, s)
        else:
            st = tg.tg_gemm_mxf8_packed(A, PA, B, PB, dptr, M, N, K, lda, ldb, ldd, s)
    elif a_fmt or b_fmt:
        st = tg.tg_gemm_mx(A, SA, B, SB, dptr, M, N, K, lda, ldsa, ldb, ldsb, ldd, a_fmt, b_fmt, s)
    else:
        st = tg.tg_gemm_mxf8(A, SA, B, SB, dptr, M, N, K, lda, ldsa, ldb, ldsb, ldd, s)
    torch.cuda.synchronize()
    full = d.cpu().numpy().view(np.uint16)[:(M + 2 * guard) * ldd].reshape(M + 2 * guard, ldd)
    win = np.array(full[guard:guard + M, guard:guard + N].view(np.float16))
    return win, full, st
