"""Host-only checks that the GPU coverage table names every kernel the
planners can choose (no device is touched: the plan entry points only
validate and choose).

1. Every case of ``planner_cases`` plans to the name it is filed under.
2. A sweep over the planners' inputs — shape classes around every tile
   threshold, tight and huge row strides, aligned and misaligned pointers,
   K multiple of 8 or not — returns only names that are in the table, and
   reaches every name the table holds.
"""
import itertools

import pytest

from planner_cases import CASES, MX_CASES, MX_FMT_SUFFIX, MXF_CASES, MXP_CASES, all_fp_names, vec_lda

tg = pytest.importorskip("dense_fp16_gemm_02_amd")

BASE = 1 << 20  # a 16-byte aligned fake device address (plans never dereference)


def _plan(fmt, M, N, K, lda, ldb, a_off=0):
    plan = tg.tg_gemm_bf16_plan if fmt == "bf16" else tg.tg_gemm_f16_plan
    st, name, tiles = plan(BASE + 2 * a_off, BASE, BASE, M, N, K, lda, ldb, N)
    assert st == tg.TG_OK
    return name


def test_every_case_plans_to_its_name():
    for name, (fmt, c) in CASES.items():
        lda, ldb = c.lds()
        assert _plan(fmt, c.M, c.N, c.K, lda, ldb, c.a_off) == name, (name, c)
    for name, c in MX_CASES.items():
        nb = c.K // 32
        ld = max(4, (nb + 3) // 4 * 4)
        st, got, _ = tg.tg_gemm_mxf8_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, ld, c.K, ld, c.N)
        assert st == tg.TG_OK and got == name, (name, c)


def test_packed_cases_plan_to_their_names():
    for name, c in MXP_CASES.items():
        st, got, _ = tg.tg_gemm_mxf8_packed_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, c.K, c.N)
        assert st == tg.TG_OK and got == name, (name, c)


def test_table_is_exactly_the_planner_universe():
    assert set(CASES) == all_fp_names()


def test_planner_sweep_stays_inside_the_table():
    Ms = [1, 2, 37, 64, 65, 100, 128, 129, 200, 256, 257, 1000, 2100, 4100]
    Ns = [131, 300, 2000, 5120, 16256, 16385, 16411, 40960]
    seen = set()
    for fmt, M, N in itertools.product(("f16", "bf16"), Ms, Ns):
        for K, a_off in ((64, 0), (128, 0), (200, 0), (250, 0), (96, 1), (2048, 0)):
            for lda in (K, vec_lda(256), vec_lda(128), vec_lda(64)):
                name = _plan(fmt, M, N, K, lda, K, a_off)
                assert name in CASES, (fmt, M, N, K, lda, a_off, name)
                seen.add(name)
    assert seen == set(CASES), sorted(set(CASES) - seen)


def test_mx_planner_sweep_stays_inside_the_table():
    seen = set()
    for M, N, K in itertools.product([1, 64, 65, 300, 2048, 2100, 8192], [600, 2060, 16256, 16400, 28672],
                                     [32, 128, 384, 512, 4096, 4192]):
        nb = K // 32
        ld = max(4, (nb + 3) // 4 * 4)
        st, name, _ = tg.tg_gemm_mxf8_plan(BASE, BASE, BASE, BASE, BASE, M, N, K, K, ld, K, ld, N)
        assert st == tg.TG_OK and name in MX_CASES, (M, N, K, name)
        seen.add(name)
        st, pname, _ = tg.tg_gemm_mxf8_packed_plan(BASE, BASE, BASE, BASE, BASE, M, N, K, K, K, N)
        assert st == tg.TG_OK and pname == name.replace("gemm_mxf8_", "gemm_mxf8p_"), (M, N, K, pname)
        seen.add(pname)
    assert seen == set(MX_CASES) | set(MXP_CASES)


def test_format_cases_plan_to_their_names():
    """tg_gemm_mx(_packed)_plan: the kernel of the E4M3 plan with the
    encodings' suffix; E4M3 on both operands is exactly tg_gemm_mxf8's plan."""
    for name, (c, fa, fb, packed) in MXF_CASES.items():
        nb = c.K // 32
        ld = max(4, (nb + 3) // 4 * 4)
        if packed:
            st, got, tiles = tg.tg_gemm_mx_packed_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, c.K,
                                                       c.N, fa, fb)
        else:
            st, got, tiles = tg.tg_gemm_mx_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, ld, c.K, ld,
                                                c.N, fa, fb)
        assert st == tg.TG_OK and got == name and tiles > 0, (name, got)
    for name, c in MX_CASES.items():
        nb = c.K // 32
        ld = max(4, (nb + 3) // 4 * 4)
        assert tg.tg_gemm_mx_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, ld, c.K, ld, c.N, 0, 0) == \
            tg.tg_gemm_mxf8_plan(BASE, BASE, BASE, BASE, BASE, c.M, c.N, c.K, c.K, ld, c.K, ld, c.N)
    assert len(MXF_CASES) == len(MX_FMT_SUFFIX) * (len(MX_CASES) + len(MXP_CASES))


@pytest.mark.parametrize("fa,fb", [(2, 0), (0, 2), (-1, 0), (0, -1), (7, 7)])
def test_unknown_encodings_are_refused(fa, fb):
    st, name, tiles = tg.tg_gemm_mx_plan(BASE, BASE, BASE, BASE, BASE, 64, 64, 64, 64, 4, 64, 4, 64, fa, fb)
    assert st == tg.TG_ERR_INVALID_ARG and name == "" and tiles == 0
    st, name, tiles = tg.tg_gemm_mx_packed_plan(BASE, BASE, BASE, BASE, BASE, 64, 64, 64, 64, 64, 64, fa, fb)
    assert st == tg.TG_ERR_INVALID_ARG and name == "" and tiles == 0
    # refused before the device is touched (this runs without a GPU)
    assert tg.tg_gemm_mx(BASE, BASE, BASE, BASE, BASE, 64, 64, 64, 64, 4, 64, 4, 64, fa, fb, None) == \
        tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_mx_packed(BASE, BASE, BASE, BASE, BASE, 64, 64, 64, 64, 64, 64, fa, fb, None) == \
        tg.TG_ERR_INVALID_ARG


def test_persistent_kernel_conditions():
    """The persistent 256x256 kernel takes direct-to-LDS launches with at
    least two tiles per compute unit (512 tiles on 256 units) and K a
    multiple of 64 from 128; everything else stays on the one-tile-per-
    workgroup kernels."""
    pers, one = "gemm_f16_256x256_w2x2_pers_dma", "gemm_f16_256x256_w2x2_dma"
    assert _plan("f16", 8192, 14336, 4096, 4096, 4096) == pers   # the linear-layer shape: 1792 tiles
    assert _plan("f16", 4096, 4096, 4096, 4096, 4096) == one     # 256 tiles: one per unit
    assert _plan("f16", 4096, 8192, 4096, 4096, 4096) == pers    # 16 x 32 = 512 tiles
    assert _plan("f16", 4096, 7936, 4096, 4096, 4096) == one     # 16 x 31 = 496 tiles
    assert _plan("f16", 8192, 14336, 128, 128, 128) == pers      # two K-tiles
    assert _plan("f16", 8192, 14336, 64, 64, 64) == one          # one K-tile
    assert _plan("f16", 8192, 14336, 4160, 4160, 4160) == pers
    assert _plan("f16", 8192, 14336, 4104, 4104, 4104) == one    # a partial K-tile
    assert _plan("bf16", 8192, 14336, 4096, 4096, 4096) == "gemm_bf16_256x256_w2x2_pers_dma"
