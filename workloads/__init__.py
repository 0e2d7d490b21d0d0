"""Seeded synthetic inputs for the fp16 GEMM D = A·Bᵀ.

This module only draws numbers; it holds none of the GEMM arithmetic and is
shared by the CPU oracle's tests, the GPU parity tests, ``smoke()`` and the
benchmark, so that both sides of every comparison see the same operands.

Shapes and value distributions follow the five workloads this library is
measured on (a single 128×128×64 tile, a ragged 1000³ case, a 4096³ square,
an 8192×14336×4096 linear layer and a 64×28672×8192 decode-like skinny
product).  Values are sampled in float64 with PCG64 and rounded to binary16
with round-to-nearest-even (numpy's ``astype(np.float16)``).

Reading of "N(0, 1/K)": the second parameter is the variance, so the weights
have standard deviation 1/sqrt(K).  "N(0,1)/4" is a standard normal divided
by four.

bfloat16 operands (for the bf16 entry point) are returned as uint16 bit
patterns: the same float64 draws, cast to float32 by numpy and cut to their
upper 16 bits (truncation: these are simply the inputs, not a rounding of
anything the GEMM computes).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_A_BASE = 1000
SEED_B_BASE = 2000
SEED_ROWS_BASE = 3000


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    N: int
    K: int
    dist_a: tuple  # ("uniform", lo, hi) | ("normal", mean, std)
    dist_b: tuple

    @property
    def flop(self) -> int:
        """Algorithmic flop count 2·M·N·K (a multiply and an add per term)."""
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """Compulsory HBM bytes: read A and B once, write D once (fp16)."""
        return 2 * (self.M * self.K + self.N * self.K + self.M * self.N)


WORKLOADS = [
    Workload(0, "single_tile_128x128x64", 128, 128, 64,
             ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0)),
    Workload(1, "ragged_1000x1000x1000", 1000, 1000, 1000,
             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0)),
    Workload(2, "square_4096x4096x4096", 4096, 4096, 4096,
             ("normal", 0.0, 0.25), ("normal", 0.0, 0.25)),
    Workload(3, "linear_8192x14336x4096", 8192, 14336, 4096,
             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / np.sqrt(4096.0))),
    Workload(4, "skinny_64x28672x8192", 64, 28672, 8192,
             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / np.sqrt(8192.0))),
]

# Shapes profiled besides the five workloads, one per kernel those do not
# reach: 2048³ runs the producer/consumer 128×128 kernel.  The same recipe
# as the linear layer (A ~ N(0,1), B ~ N(0,1/K)).
EXTRA_WORKLOADS = [
    Workload(5, "mid_2048x2048x2048", 2048, 2048, 2048,
             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / np.sqrt(2048.0))),
]

BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def _draw64(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.standard_normal(size=shape) * dist[2] + dist[1]
    raise ValueError(f"unknown distribution {dist!r}")


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 draws → bfloat16 bit patterns (float32 cast, low half cut)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _draw(rng: np.random.Generator, shape, dist, dtype: str = "f16") -> np.ndarray:
    x = _draw64(rng, shape, dist)
    return to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16)


def make_inputs(w: Workload, lda: Optional[int] = None, ldb: Optional[int] = None,
                dtype: str = "f16"):
    """Return (A, B) of shape (M, lda) and (N, ldb): float16 arrays, or
    uint16 bfloat16 bit patterns with ``dtype="bf16"``.

    The logical operands are A[:, :K] and B[:, :K]; padding columns (when
    lda > K or ldb > K) are filled with NaN so that any read past K shows up
    as NaN in D.
    """
    lda = w.K if lda is None else lda
    ldb = w.K if ldb is None else ldb
    a = _draw(np.random.Generator(np.random.PCG64(SEED_A_BASE + w.index)), (w.M, w.K), w.dist_a, dtype)
    b = _draw(np.random.Generator(np.random.PCG64(SEED_B_BASE + w.index)), (w.N, w.K), w.dist_b, dtype)
    if lda != w.K:
        a = pad_columns(a, lda)
    if ldb != w.K:
        b = pad_columns(b, ldb)
    return a, b


BF16_NAN = np.uint16(0x7fc0)


def pad_columns(x: np.ndarray, ld: int, fill=np.nan) -> np.ndarray:
    """Copy a (rows, K) matrix into a (rows, ld) buffer, padding with ``fill``
    (NaN; for uint16 bf16 bit arrays the bf16 NaN pattern)."""
    rows, k = x.shape
    if ld < k:
        raise ValueError("leading dimension smaller than the row length")
    if x.dtype == np.uint16:
        out = np.full((rows, ld), BF16_NAN if np.isnan(fill) else fill, dtype=np.uint16)
    else:
        out = np.full((rows, ld), fill, dtype=np.float16)
    out[:, :k] = x
    return out


def sample_rows(w: Workload, count: int = 64) -> np.ndarray:
    """Rows of D checked for the large workloads: ``count`` seeded random rows
    (without replacement) plus the first and last row, sorted and unique."""
    rng = np.random.default_rng(SEED_ROWS_BASE + w.index)
    picked = rng.choice(w.M, size=min(count, w.M), replace=False)
    rows = np.unique(np.concatenate([picked, [0, w.M - 1]]))
    return rows.astype(np.int64)


def random_f16(seed: int, shape, dist=("normal", 0.0, 1.0)) -> np.ndarray:
    """Small helper for ad-hoc seeded operands (edge-case tests)."""
    return _draw(np.random.Generator(np.random.PCG64(seed)), shape, dist)


def random_bf16(seed: int, shape, dist=("normal", 0.0, 1.0)) -> np.ndarray:
    """Seeded bfloat16 operands as uint16 bit patterns."""
    return _draw(np.random.Generator(np.random.PCG64(seed)), shape, dist, "bf16")


def index_pattern(M: int, N: int, K: int):
    """Integer-valued operands whose products are exact in fp32 and fp16 for
    K <= 341: A[i,k] = ((i + 2k) mod 5) - 2 and B[j,k] = ((3j + k) mod 7) - 3,
    so |D| <= 6K.  Any swapped fragment, swizzle or tile offset changes D."""
    i = np.arange(M)[:, None]
    j = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    a = (((i + 2 * k) % 5) - 2).astype(np.float16)
    b = (((3 * j + k) % 7) - 3).astype(np.float16)
    return a, b


def small_int_pattern(M: int, N: int, K: int, dtype: str = "f16"):
    """Operands in {-1, 0, 1}: A[i,k] = ((i + 2k) mod 3) - 1, B[j,k] =
    ((2j + k) mod 3) - 1, so |D| <= K and D is exact in bfloat16 for K <= 256
    (and in binary16 for K <= 2048)."""
    i = np.arange(M)[:, None]
    j = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    a = (((i + 2 * k) % 3) - 1).astype(np.float64)
    b = (((2 * j + k) % 3) - 1).astype(np.float64)
    if dtype == "bf16":
        return to_bf16_bits(a), to_bf16_bits(b)
    return a.astype(np.float16), b.astype(np.float16)


# ------------------------------------------------------------ block-scaled FP8
#
# Operands of the block-scaled FP8 entry point: FP8 E4M3 codes (uint8) with
# one UE8M0 scale byte per MX_BLOCK consecutive K elements of every row.
# Synthetic data are drawn like the fp16 operands (same seeds and
# distributions) and then encoded the way OCP MX encodes a float block: the
# block's shared exponent is floor(log2(max |x|)) minus 8 (the largest E4M3
# exponent; 448 = 1.75·2^8), clamped to [-127, 127] (an all-zero block takes
# -127), and every element x / 2^exp is rounded to the nearest E4M3 value,
# ties to the even code, saturating at ±448.  This is input preparation only:
# the GEMM consumes the codes and scales as given.  E5M2 operands (OCP MX's
# second FP8 encoding) are encoded the same way with the shared exponent
# floor(log2(max |x|)) minus 15 (57344 = 1.75·2^15) and saturation at
# ±57344.

MX_BLOCK = 32
MX_NAN = np.uint8(0x7f)


def _e4m3_grid():
    """The 127 non-negative finite E4M3 values in code order (increasing)."""
    codes = np.arange(0x7f, dtype=np.int64)
    e, f = codes >> 3, codes & 7
    vals = np.where(e == 0, f * 2.0 ** -9, (8 + f) * 2.0 ** (e - 10))
    return vals, codes.astype(np.uint8)


_E4M3_VALS, _E4M3_CODES = _e4m3_grid()


def _e5m2_grid():
    """The 124 non-negative finite E5M2 values in code order (increasing)."""
    codes = np.arange(0x7c, dtype=np.int64)
    e, f = codes >> 2, codes & 3
    vals = np.where(e == 0, f * 2.0 ** -16, (4 + f) * 2.0 ** (e - 17))
    return vals, codes.astype(np.uint8)


_E5M2_VALS, _E5M2_CODES = _e5m2_grid()


def _encode_grid(q, vals, codes, top, top_code):
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), top)
    i = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 2)
    lo, hi = vals[i], vals[i + 1]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & ((codes[i] & 1) == 1))
    c = np.where(up, codes[i + 1], codes[i]).astype(np.uint8)
    c = np.where(a >= top, np.uint8(top_code), c)
    return np.where((q < 0) & (c != 0), c | np.uint8(0x80), c).astype(np.uint8)


def encode_e5m2(q: np.ndarray) -> np.ndarray:
    """Nearest E5M2 code (ties to the even code), saturating at ±57344."""
    return _encode_grid(q, _E5M2_VALS, _E5M2_CODES, 57344.0, 0x7b)


def encode_e4m3(q: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code), saturating at ±448."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), 448.0)
    i = np.clip(np.searchsorted(_E4M3_VALS, a, side="right") - 1, 0, len(_E4M3_VALS) - 2)
    lo, hi = _E4M3_VALS[i], _E4M3_VALS[i + 1]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & ((_E4M3_CODES[i] & 1) == 1))
    c = np.where(up, _E4M3_CODES[i + 1], _E4M3_CODES[i]).astype(np.uint8)
    c = np.where(a >= 448.0, np.uint8(0x7e), c)
    return np.where((q < 0) & (c != 0), c | np.uint8(0x80), c).astype(np.uint8)


def mx_quantize(x: np.ndarray, fmt: str = "e4m3"):
    """Encode a float64 (rows, K) matrix as (codes (rows, K) uint8, scales
    (rows, ceil(K/32)) uint8) with the shared-exponent recipe above, in the
    element encoding ``fmt`` ("e4m3" or "e5m2")."""
    if fmt not in ("e4m3", "e5m2"):
        raise ValueError("fmt is 'e4m3' or 'e5m2'")
    top_exp = 8 if fmt == "e4m3" else 15
    x = np.asarray(x, dtype=np.float64)
    rows, K = x.shape
    nb = (K + MX_BLOCK - 1) // MX_BLOCK
    padded = np.zeros((rows, nb * MX_BLOCK))
    padded[:, :K] = x
    blocks = padded.reshape(rows, nb, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - top_exp, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    enc = encode_e4m3 if fmt == "e4m3" else encode_e5m2
    codes = enc(blocks / np.exp2(e)[:, :, None]).reshape(rows, nb * MX_BLOCK)[:, :K]
    return np.ascontiguousarray(codes), (e + 127).astype(np.uint8)


def make_mx_inputs(w: Workload, a_fmt: str = "e4m3", b_fmt: str = "e4m3"):
    """Block-scaled FP8 operands for workload ``w``: (A, SA, B, SB), the same
    float64 draws as ``make_inputs`` encoded with ``mx_quantize`` (element
    encodings a_fmt, b_fmt)."""
    a = _draw64(np.random.Generator(np.random.PCG64(SEED_A_BASE + w.index)), (w.M, w.K), w.dist_a)
    b = _draw64(np.random.Generator(np.random.PCG64(SEED_B_BASE + w.index)), (w.N, w.K), w.dist_b)
    qa, sa = mx_quantize(a, a_fmt)
    del a
    qb, sb = mx_quantize(b, b_fmt)
    return qa, sa, qb, sb


def random_mx(seed: int, rows: int, K: int, scale_lo: int = 120, scale_hi: int = 134, fmt: str = "e4m3"):
    """Seeded random FP8 codes (every finite code of the encoding ``fmt``,
    "e4m3" or "e5m2", both signs; NaN and infinity codes excluded) with random
    scale bytes in [scale_lo, scale_hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 256, size=(rows, K)).astype(np.uint8)
    if fmt == "e4m3":
        codes = np.where((codes & 0x7f) == 0x7f, codes ^ np.uint8(1), codes).astype(np.uint8)
    elif fmt == "e5m2":  # exponent field 31 (infinity, NaN) moved down to 30
        codes = np.where((codes & 0x7c) == 0x7c, codes ^ np.uint8(0x04), codes).astype(np.uint8)
    else:
        raise ValueError("fmt is 'e4m3' or 'e5m2'")
    scales = rng.integers(scale_lo, scale_hi + 1, size=(rows, (K + MX_BLOCK - 1) // MX_BLOCK)).astype(np.uint8)
    return codes, scales


def pad_bytes(x: np.ndarray, ld: int, fill: int = 0x7f) -> np.ndarray:
    """Copy a (rows, n) uint8 matrix into a (rows, ld) buffer padded with
    ``fill`` (the E4M3 NaN code by default, which is also a NaN-sized scale
    once it reaches 0xff)."""
    rows, n = x.shape
    if ld < n:
        raise ValueError("leading dimension smaller than the row length")
    out = np.full((rows, ld), fill, dtype=np.uint8)
    out[:, :n] = x
    return out
