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


def to_dev(x: np.ndarray, offset_elems: int = 0):
    """Copy a 2-D fp16 array into a device buffer starting `offset_elems`
    elements past a 256-byte aligned allocation (offset 1 misaligns it)."""
    import torch

    flat = np.ascontiguousarray(x, dtype=np.float16).reshape(-1)
    buf = torch.empty(flat.size + offset_elems + 8, dtype=torch.float16, device="cuda:0")
    buf.fill_(float("nan"))
    if flat.size:
        buf[offset_elems:offset_elems + flat.size].copy_(torch.from_numpy(flat))
    return buf, buf.data_ptr() + 2 * offset_elems


def run(a: np.ndarray, b: np.ndarray, M: int, N: int, K: int, *, ldd: int | None = None,
        guard: int = 0, a_off: int = 0, b_off: int = 0, d_off: int = 0, stream=None,
        label: str = ""):
    """D = A·Bᵀ on the GPU.  a is (M, lda) and b is (N, ldb) fp16 (padding
    columns beyond K are passed through untouched).  D lives in a buffer of
    (M + 2·guard) rows × ldd_total columns filled with SENTINEL, with the
    window at (guard, guard).  Returns (D window as fp16 (M, N), full buffer
    as uint16 for guard checks, status)."""
    import torch

    import dense_fp16_gemm_02_amd as tg

    lda = a.shape[1] if a.ndim == 2 and a.shape[1] else max(K, 1)
    ldb = b.shape[1] if b.ndim == 2 and b.shape[1] else max(K, 1)
    ldd = (N + 2 * guard) if ldd is None else ldd
    rows_total = M + 2 * guard
    a_buf, a_ptr = to_dev(a, a_off)
    b_buf, b_ptr = to_dev(b, b_off)
    d_buf = torch.full((rows_total * ldd + d_off + 8,), 0, dtype=torch.int16, device="cuda:0")
    d_buf.fill_(SENTINEL)
    d_ptr = d_buf.data_ptr() + 2 * (d_off + guard * ldd + guard)
    s = stream if stream is not None else torch.cuda.current_stream()
    say(f"{label} M={M} N={N} K={K} lda={lda} ldb={ldb} ldd={ldd} guard={guard} "
        f"offs=({a_off},{b_off},{d_off})")
    st = tg.tg_gemm_f16(a_ptr, b_ptr, d_ptr, M, N, K, lda, ldb, ldd, s)
    s.synchronize()
    torch.cuda.synchronize()
    full = d_buf.cpu().numpy().view(np.uint16)[d_off:d_off + rows_total * ldd].reshape(rows_total, ldd)
    win = full[guard:guard + M, guard:guard + N].view(np.float16)
    del a_buf, b_buf
    return np.array(win), full, st


def guard_intact(full: np.ndarray, M: int, N: int, guard: int) -> bool:
    mask = np.ones(full.shape, dtype=bool)
    mask[guard:guard + M, guard:guard + N] = False
    return bool(np.all(full[mask] == SENTINEL))
