"""One launch per kernel instantiation the public entry points can choose.

The planners (tg_gemm_f16_plan, tg_gemm_bf16_plan, tg_gemm_mxf8_plan) pick a
tile and a load path from the shape, the leading dimensions and the operand
alignment.  ``CASES`` maps every kernel name they can return to one problem
that plans to it; ``tests/test_planner_cpu.py`` checks that mapping on the
host and that a sweep over the planners' inputs returns no other name, and
``tests/test_gpu_planner_coverage.py`` runs every case on the GPU against the
oracle, element by element and bit for bit (integer-valued operands make
every sum exact).

Load paths: "dma" (direct-to-LDS, 16-byte aligned operands, K, lda, ldb
multiples of 8, in-tile byte offsets below 2^31), "vec" (the same alignment
but a row stride so large that a tile's byte offsets pass 2^31: 16-byte
loads through registers) and "scalar" (anything not 16-byte aligned, or K /
lda / ldb not multiples of 8: element-wise loads).
"""
from __future__ import annotations

from dataclasses import dataclass

# smallest multiple of 8 with (rows - 1)·lda·2 + 128 >= 2^31 - 1: tiles of
# `rows` rows then address past 32 bits and take the register path
def vec_lda(rows: int) -> int:
    limit = (1 << 31) - 1 - 128
    ld = limit // (2 * (rows - 1)) + 1
    return (ld + 7) // 8 * 8


@dataclass(frozen=True)
class Case:
    M: int
    N: int
    K: int
    lda: int = 0      # 0: tight (K)
    ldb: int = 0
    a_off: int = 0    # element offset of A from a 256-byte boundary (1 misaligns)

    def lds(self):
        return self.lda or self.K, self.ldb or self.K


# (tile, path) -> Case.  The integer patterns keep sums exact: the fp16 index
# pattern for K <= 341, else {-1, 0, 1} (|D| <= K <= 2048); the bf16 {-1, 0, 1}
# pattern, whose fp32 sums stay exact integers, rounded once on both sides.
_F16_BF16 = {
    # column strips, M <= 64 / 128 / 256 with at least 128 strips of 128 columns
    ("64x128_w1x4", "dma"): Case(37, 16411, 200),
    ("64x128_w1x4", "vec"): Case(2, 16400, 64, lda=vec_lda(64)),
    ("64x128_w1x4", "scalar"): Case(64, 16411, 250),
    ("128x128_w2x2_strip", "dma"): Case(100, 16411, 200),
    ("128x128_w2x2_strip", "vec"): Case(66, 16385, 64, lda=vec_lda(128)),
    ("128x128_w2x2_strip", "scalar"): Case(128, 16390, 96, a_off=1),
    ("256x128_w2x2", "dma"): Case(200, 16400, 200),
    ("256x128_w2x2", "vec"): Case(130, 16385, 64, lda=vec_lda(256)),
    ("256x128_w2x2", "scalar"): Case(256, 16411, 250),
    # 256x256 from 160 tiles, 128x128 from 80, else 64x64
    ("256x256_w2x2", "dma"): Case(4100, 4200, 200),
    ("256x256_w2x2", "vec"): Case(257, 40960, 64, lda=vec_lda(256)),
    ("256x256_w2x2", "scalar"): Case(4100, 4200, 250),
    # persistent 256x256 (at least 2 tiles per compute unit, K a multiple of
    # 64 from 128): 561 tiles, so each of the 256 workgroups crosses 1-2 tile
    # boundaries inside its K-tile stream; ragged M and N
    ("256x256_w2x2_pers", "dma"): Case(4100, 8200, 192),
    # 128x128 on the direct-to-LDS path: the producer/consumer kernel
    ("128x128_w2x2_ws", "dma"): Case(2100, 2000, 200),
    ("128x128_w2x2", "vec"): Case(129, 5120, 64, lda=vec_lda(128)),
    ("128x128_w2x2", "scalar"): Case(1000, 2000, 250),
    # 64x32 on the direct-to-LDS path: at most 128 tiles of 64x64 and K >= 2048
    ("64x32_w2x2", "dma"): Case(64, 3584, 2048),
    ("64x64_w2x2", "dma"): Case(1000, 1000, 200),
    ("64x64_w2x2", "vec"): Case(2, 300, 64, lda=17_100_000),
    ("64x64_w2x2", "scalar"): Case(97, 131, 250),
}

CASES: dict[str, tuple[str, Case]] = {}
for (tile, path), case in _F16_BF16.items():
    for dt, prefix in (("f16", "gemm_f16_"), ("bf16", "gemm_bf16_")):
        CASES[f"{prefix}{tile}_{path}"] = (dt, case)

# block-scaled FP8: the 64x128 kernel (small M or few tiles) and the 256x256
# kernel with scale words in groups of four K-tiles (4 divides the K-tile
# count) or in pairs
MX_CASES: dict[str, Case] = {
    "gemm_mxf8_64x128_w1x4_dma": Case(64, 16400, 1024),
    "gemm_mxf8_256x256_w2x2_g4_dma": Case(2100, 2060, 512),
    "gemm_mxf8_256x256_w2x2_g2_dma": Case(2100, 2060, 384),
}

# the same kernels reading scales in the packed layout (tg_gemm_mxf8_packed)
MXP_CASES: dict[str, Case] = {n.replace("gemm_mxf8_", "gemm_mxf8p_"): c for n, c in MX_CASES.items()}

# the other element encodings (tg_gemm_mx, tg_gemm_mx_packed): (A, B) encodings
# (0 E4M3, 1 E5M2) and the name suffix they add
MX_FMT_SUFFIX = {(1, 0): "_e5m2xe4m3", (0, 1): "_e4m3xe5m2", (1, 1): "_e5m2"}
MXF_CASES: dict[str, tuple] = {
    n + sfx: (c, fa, fb, n in MXP_CASES)
    for n, c in list(MX_CASES.items()) + list(MXP_CASES.items())
    for (fa, fb), sfx in MX_FMT_SUFFIX.items()
}

TILES = sorted({t for t, _ in _F16_BF16})
PATHS = ("dma", "vec", "scalar")
DMA_ONLY = {"256x256_w2x2_pers", "128x128_w2x2_ws", "64x32_w2x2"}  # kernels only on the direct-to-LDS path
NO_DMA = {"128x128_w2x2"}  # kernels whose direct-to-LDS form is another kernel


def all_fp_names() -> set:
    """Every name the fp16/bf16 planners can return."""
    return {f"gemm_{dt}_{t}_{p}" for dt in ("f16", "bf16") for t in TILES for p in PATHS
            if (p == "dma" or t not in DMA_ONLY) and not (p == "dma" and t in NO_DMA)}
