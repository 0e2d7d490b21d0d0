"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/*.h declares, rejects bad arguments before touching a
device, and plans kernels for the measured workloads."""
import ctypes
import os
import re

import pytest

import workloads

tg = pytest.importorskip("dense_fp16_gemm_02_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(INCLUDE)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tg_\w+)\s*\(", text, flags=re.M)
    return names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(tg.lib_path())
    names = declared_functions()
    assert "tg_gemm_f16" in names and "tg_status_string" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"


def test_library_is_built_for_gfx950():
    with open(tg.lib_path(), "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


FAKE = 1 << 20  # a non-NULL pointer value; validation rejects before any use


@pytest.mark.parametrize("args", [
    (FAKE, FAKE, FAKE, -1, 4, 4, 4, 4, 4),   # negative M
    (FAKE, FAKE, FAKE, 4, -1, 4, 4, 4, 4),   # negative N
    (FAKE, FAKE, FAKE, 4, 4, -1, 4, 4, 4),   # negative K
    (FAKE, FAKE, FAKE, 4, 4, 8, 7, 8, 4),    # lda < K
    (FAKE, FAKE, FAKE, 4, 4, 8, 8, 7, 4),    # ldb < K
    (FAKE, FAKE, FAKE, 4, 4, 8, 8, 8, 3),    # ldd < N
    (None, FAKE, FAKE, 4, 4, 8, 8, 8, 4),    # NULL A with elements
    (FAKE, None, FAKE, 4, 4, 8, 8, 8, 4),    # NULL B with elements
    (FAKE, FAKE, None, 4, 4, 8, 8, 8, 4),    # NULL D with elements
])
def test_invalid_arguments_rejected_without_launch(args):
    assert tg.tg_gemm_f16(*args, None) == tg.TG_ERR_INVALID_ARG
    st, name, tiles = tg.tg_gemm_f16_plan(*args)
    assert st == tg.TG_ERR_INVALID_ARG and name == "" and tiles == 0


def test_too_large_rejected():
    big = 1 << 31
    assert tg.tg_gemm_f16(FAKE, FAKE, FAKE, big, 4, 4, 4, 4, 4, None) == tg.TG_ERR_TOO_LARGE
    assert tg.tg_gemm_f16(FAKE, FAKE, FAKE, 4, 4, 4, big, 4, 4, None) == tg.TG_ERR_TOO_LARGE


def test_empty_problems_are_noops():
    # M == 0 or N == 0: OK with nothing launched; matrices without elements
    # may be NULL
    assert tg.tg_gemm_f16(None, FAKE, None, 0, 5, 3, 3, 3, 5, None) == tg.TG_OK
    assert tg.tg_gemm_f16(FAKE, None, None, 5, 0, 3, 3, 3, 0, None) == tg.TG_OK
    assert tg.tg_gemm_f16(None, None, None, 0, 0, 0, 0, 0, 0, None) == tg.TG_OK
    assert tg.tg_gemm_f16_plan(None, FAKE, None, 0, 5, 3, 3, 3, 5) == (tg.TG_OK, "", 0)


def test_status_strings():
    for st in (tg.TG_OK, tg.TG_ERR_INVALID_ARG, tg.TG_ERR_LAUNCH, tg.TG_ERR_DEVICE,
               tg.TG_ERR_TOO_LARGE):
        s = tg.tg_status_string(st)
        assert s and s != "unknown status"
    assert tg.tg_status_string(12345) == "unknown status"


def test_plans_for_workloads():
    for w in workloads.WORKLOADS:
        st, name, tiles = tg.tg_gemm_f16_plan(FAKE, FAKE, FAKE, w.M, w.N, w.K, w.K, w.K, w.N)
        assert st == tg.TG_OK and name.startswith("gemm_f16_") and name.endswith("_dma")
        assert tiles > 0
    # misaligned pointer or K % 8 != 0 takes the element-wise path
    st, name, _ = tg.tg_gemm_f16_plan(FAKE + 2, FAKE, FAKE, 64, 64, 64, 64, 64, 64)
    assert name.endswith("_scalar")
    st, name, _ = tg.tg_gemm_f16_plan(FAKE, FAKE, FAKE, 64, 64, 60, 60, 60, 64)
    assert name.endswith("_scalar")


@pytest.mark.parametrize("M,N,K,tile,tiles", [
    (64, 28672, 8192, "64x128", 224),     # decode-like: one strip row, B streamed once
    (1, 16385, 64, "64x128", 129),
    (128, 28672, 8192, "128x128", 224),
    (256, 28672, 8192, "256x128", 224),
    (64, 4096, 8192, "64x32", 128),       # too few strips to fill the chip; long K: 64x32 tiles
    (64, 4096, 1024, "64x64", 64),        # the same with short K
    (8192, 14336, 4096, "256x256", 1792),
    (4096, 4096, 4096, "256x256", 256),
    (2048, 2048, 2048, "128x128", 256),
    (1000, 1000, 1000, "64x64", 256),
])
def test_tile_choice(M, N, K, tile, tiles):
    st, name, g = tg.tg_gemm_f16_plan(FAKE, FAKE, FAKE, M, N, K, K, K, N)
    assert st == tg.TG_OK and name.startswith(f"gemm_f16_{tile}_") and g == tiles


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    import importlib
    import dense_fp16_gemm_02_amd as pkg
    monkeypatch.setattr(pkg, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pkg, "_lib", None)
    with pytest.raises(ImportError):
        pkg.load()
    importlib.reload(pkg)


def test_bf16_plans_and_validation():
    for w in workloads.WORKLOADS:
        st, name, tiles = tg.tg_gemm_bf16_plan(FAKE, FAKE, FAKE, w.M, w.N, w.K, w.K, w.K, w.N)
        st16, name16, tiles16 = tg.tg_gemm_f16_plan(FAKE, FAKE, FAKE, w.M, w.N, w.K, w.K, w.K, w.N)
        assert st == tg.TG_OK and name == name16.replace("gemm_f16_", "gemm_bf16_")
        assert tiles == tiles16
    assert tg.tg_gemm_bf16(FAKE, FAKE, FAKE, 4, 4, 8, 4, 8, 4, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_bf16(FAKE, FAKE, FAKE, 1 << 31, 4, 4, 4, 4, 4, None) == tg.TG_ERR_TOO_LARGE
    assert tg.tg_gemm_bf16(None, None, None, 0, 0, 0, 0, 0, 0, None) == tg.TG_OK


def test_mxf8_plans_and_validation():
    """Host-side checks of the block-scaled entry point: plans for the
    workloads whose K is whole 32-element blocks, and every rejection rule
    (none of these calls reaches a device)."""
    for w in workloads.WORKLOADS:
        nb = (w.K // 32 + 3) // 4 * 4
        st, name, tiles = tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, w.M, w.N, w.K, w.K, nb, w.K, nb, w.N)
        if w.K % 32:
            assert st == tg.TG_ERR_LAYOUT and name == "" and tiles == 0
            continue
        big_tiles = ((w.M + 255) // 256) * ((w.N + 255) // 256)
        if (w.M <= 64 and (w.N + 127) // 128 >= 128) or big_tiles < 64:  # 64x128 tiles
            assert st == tg.TG_OK and name == "gemm_mxf8_64x128_w1x4_dma"
            assert tiles == ((w.M + 63) // 64) * ((w.N + 127) // 128)
        else:
            group = "g4" if ((w.K + 127) // 128) % 4 == 0 else "g2"
            assert st == tg.TG_OK and name == f"gemm_mxf8_256x256_w2x2_{group}_dma"
            assert tiles == ((w.M + 255) // 256) * ((w.N + 255) // 256)
    # the strip needs M <= 64 and at least 128 strips
    assert tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 16384, 128, 128, 4, 128, 4, 16384)[1] == \
        "gemm_mxf8_64x128_w1x4_dma"
    assert tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 16384, 128, 128, 4, 128, 4, 16384)[1] == \
        "gemm_mxf8_256x256_w2x2_g2_dma"
    assert tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 16256, 128, 128, 4, 128, 4, 16256)[1] == \
        "gemm_mxf8_256x256_w2x2_g2_dma"
    # and problems with fewer than 64 tiles of 256x256 take 64x128 tiles
    assert tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 1792, 128, 128, 4, 128, 4, 1792)[1:] == \
        ("gemm_mxf8_64x128_w1x4_dma", 32 * 14)
    assert tg.tg_gemm_mxf8_plan(FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 2048, 128, 128, 4, 128, 4, 2048)[1] == \
        "gemm_mxf8_256x256_w2x2_g2_dma"
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 128, 128, 4, 128, 4, 64)
    assert tg.tg_gemm_mxf8_plan(*ok)[0] == tg.TG_OK

    def with_(**kw):
        names = ["A", "SA", "B", "SB", "D", "M", "N", "K", "lda", "ldsa", "ldb", "ldsb", "ldd"]
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return tg.tg_gemm_mxf8_plan(*args)[0], tg.tg_gemm_mxf8(*args, None)

    for kw, want in [({"K": 100, "lda": 128, "ldb": 128}, tg.TG_ERR_LAYOUT),
                     ({"lda": 136}, tg.TG_ERR_LAYOUT), ({"ldb": 200}, tg.TG_ERR_LAYOUT),
                     ({"ldsa": 6}, tg.TG_ERR_LAYOUT), ({"ldsb": 5}, tg.TG_ERR_LAYOUT),
                     ({"A": FAKE + 8}, tg.TG_ERR_LAYOUT), ({"B": FAKE + 4}, tg.TG_ERR_LAYOUT),
                     ({"SA": FAKE + 2}, tg.TG_ERR_LAYOUT), ({"SB": FAKE + 1}, tg.TG_ERR_LAYOUT),
                     ({"lda": 112}, tg.TG_ERR_INVALID_ARG), ({"ldsa": 3}, tg.TG_ERR_INVALID_ARG),
                     ({"ldd": 63}, tg.TG_ERR_INVALID_ARG), ({"M": -1}, tg.TG_ERR_INVALID_ARG),
                     ({"SA": None}, tg.TG_ERR_INVALID_ARG), ({"SB": None}, tg.TG_ERR_INVALID_ARG),
                     ({"D": None}, tg.TG_ERR_INVALID_ARG),
                     ({"M": 1 << 31}, tg.TG_ERR_TOO_LARGE), ({"lda": 1 << 24}, tg.TG_ERR_TOO_LARGE),
                     ({"ldsb": 1 << 23}, tg.TG_ERR_TOO_LARGE)]:
        assert with_(**kw) == (want, want), kw
    # empty problems launch nothing and need no pointers
    assert tg.tg_gemm_mxf8(None, None, None, None, None, 0, 0, 0, 0, 0, 0, 0, 0, None) == tg.TG_OK
    assert tg.tg_gemm_mxf8_plan(None, None, FAKE, FAKE, None, 0, 7, 64, 64, 4, 64, 4, 7) == (tg.TG_OK, "", 0)
    assert tg.tg_status_string(tg.TG_ERR_LAYOUT) != "unknown status"


def test_torch_wrapper_refuses_cpu_tensors():
    """gemm() hands device pointers to the kernels: host tensors are refused
    before any call reaches the library."""
    torch = pytest.importorskip("torch")
    A = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensors"):
        tg.gemm(A, A)
    with pytest.raises(TypeError):
        tg.gemm(A, A.float())


def test_ceiling_codes_and_validation():
    """The instruction codes of tg_mfma_ceiling agree with include/tg_ceiling.h,
    and bad arguments of both measurement entry points are rejected before a
    device is touched."""
    text = open(os.path.join(INCLUDE, "tg_ceiling.h")).read()
    codes = dict(re.findall(r"#define (TG_MFMA_\w+) (\d+)", text))
    assert len(codes) == 4
    for name, value in codes.items():
        assert getattr(tg, name) == int(value), name
    ok = dict(A=FAKE, a=1 << 16, B=FAKE, b=1 << 16, w=1, it=4, wg=256, out=FAKE)
    bad = [dict(shape=99), dict(shape=0),
           dict(shape=tg.TG_MFMA_F16_16X16X32, a=12), dict(shape=tg.TG_MFMA_BF16_16X16X32, b=4),
           dict(shape=tg.TG_MFMA_MXF8_32X32X64, a=48), dict(shape=tg.TG_MFMA_MXF8_32X32X64, b=16),
           dict(shape=tg.TG_MFMA_F16_32X32X16, A=FAKE + 8), dict(shape=tg.TG_MFMA_MXF8_32X32X64, B=FAKE + 4),
           dict(shape=tg.TG_MFMA_F16_16X16X32, A=None), dict(shape=tg.TG_MFMA_F16_16X16X32, out=None),
           dict(shape=tg.TG_MFMA_F16_16X16X32, w=2), dict(shape=tg.TG_MFMA_F16_16X16X32, it=0),
           dict(shape=tg.TG_MFMA_MXF8_32X32X64, wg=0)]
    for kw in bad:
        p = {**ok, **kw}
        st = tg.tg_mfma_ceiling(p["shape"], p["A"], p["a"], p["B"], p["b"], p["w"], p["it"], p["wg"], p["out"])
        assert st == tg.TG_ERR_INVALID_ARG, kw
    for src, nbytes, wg, out in [(None, 1 << 20, 256, FAKE), (FAKE, 8, 256, FAKE), (FAKE, 1000, 256, FAKE),
                                 (FAKE + 4, 1 << 20, 256, FAKE), (FAKE, 1 << 20, 0, FAKE),
                                 (FAKE, 1 << 20, 256, None)]:
        assert tg.tg_hbm_read_ceiling(src, nbytes, wg, out) == tg.TG_ERR_INVALID_ARG


def test_packed_scale_entry_points_validation():
    """The packed-scale entry points: buffer sizes, kernel names, and every
    rejection before a device is touched."""
    assert tg.tg_mx_packed_bytes(0, 4096) == 0
    assert tg.tg_mx_packed_bytes(1, 32) == 512
    assert tg.tg_mx_packed_bytes(32, 512) == 512
    assert tg.tg_mx_packed_bytes(33, 512) == 1024
    assert tg.tg_mx_packed_bytes(64, 544) == 2048
    assert tg.tg_mx_packed_bytes(8192, 4096) == 256 * 8 * 512
    for rows, K in [(-1, 32), (4, 33), (4, -32), (1 << 31, 32)]:
        assert tg.tg_mx_packed_bytes(rows, K) == -1
    names = {}
    for w in workloads.WORKLOADS:
        K = w.K - w.K % 32
        st, name, tiles = tg.tg_gemm_mxf8_packed_plan(FAKE, FAKE, FAKE, FAKE, FAKE, w.M, w.N, K, K, K, w.N)
        assert st == tg.TG_OK
        names[w.name] = name
    assert names["linear_8192x14336x4096"] == "gemm_mxf8p_256x256_w2x2_g4_dma"
    assert names["skinny_64x28672x8192"] == "gemm_mxf8p_64x128_w1x4_dma"
    ok = dict(A=FAKE, SA=FAKE, B=FAKE, SB=FAKE, D=FAKE, M=300, N=300, K=128, lda=128, ldb=128, ldd=300)
    for kw, want in [({"K": 100, "lda": 112, "ldb": 112}, tg.TG_ERR_LAYOUT), ({"lda": 136}, tg.TG_ERR_LAYOUT),
                     ({"SA": FAKE + 4}, tg.TG_ERR_LAYOUT), ({"SB": FAKE + 8}, tg.TG_ERR_LAYOUT),
                     ({"A": FAKE + 8}, tg.TG_ERR_LAYOUT), ({"M": -1}, tg.TG_ERR_INVALID_ARG),
                     ({"lda": 96}, tg.TG_ERR_INVALID_ARG), ({"ldd": 299}, tg.TG_ERR_INVALID_ARG),
                     ({"SA": None}, tg.TG_ERR_INVALID_ARG), ({"D": None}, tg.TG_ERR_INVALID_ARG),
                     ({"K": 1 << 27, "lda": 1 << 27, "ldb": 1 << 27}, tg.TG_ERR_TOO_LARGE),
                     ({"M": 1 << 31}, tg.TG_ERR_TOO_LARGE)]:
        p = {**ok, **kw}
        args = [p[k] for k in ("A", "SA", "B", "SB", "D", "M", "N", "K", "lda", "ldb", "ldd")]
        assert tg.tg_gemm_mxf8_packed(*args, None) == want, kw
        st, name, tiles = tg.tg_gemm_mxf8_packed_plan(*args)
        assert st == want and name == "" and tiles == 0, kw
    # the pack: argument checks, and nothing to do for empty matrices
    assert tg.tg_mx_pack_scales(FAKE, 4, 33, 4, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_mx_pack_scales(FAKE, 4, 128, 3, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_mx_pack_scales(None, 4, 128, 4, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_mx_pack_scales(FAKE, -1, 128, 4, FAKE, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_mx_pack_scales(FAKE, 4, 128, 4, FAKE + 4, None) == tg.TG_ERR_LAYOUT
    assert tg.tg_mx_pack_scales(FAKE, 1 << 31, 128, 4, FAKE, None) == tg.TG_ERR_TOO_LARGE
    assert tg.tg_mx_pack_scales(None, 0, 128, 4, None, None) == tg.TG_OK


def test_xcd_stamps_validation():
    """The stamping entry point runs only problems that plan to the
    persistent kernel, with room for three words per workgroup; everything
    else is refused before a device is touched."""
    M, N, K = 8192, 14336, 4096  # persistent: 1792 tiles, at most 256 workgroups
    big = 3 * 4096
    for kw in [dict(M=128, N=128, K=64), dict(M=1000, N=1000, K=1000), dict(M=4096, N=4096, K=4096),
               dict(K=4000), dict(stamps=None), dict(stamps_len=3), dict(M=0), dict(M=-1), dict(lda=8)]:
        p = {**dict(M=M, N=N, K=K, lda=None, stamps=FAKE, stamps_len=big), **kw}
        lda = p["lda"] if p["lda"] is not None else p["K"]
        st, wg = tg.tg_gemm_f16_xcd_stamps(FAKE, FAKE, FAKE, p["M"], p["N"], p["K"], lda, p["K"], p["N"],
                                           p["stamps"], p["stamps_len"])
        assert st == tg.TG_ERR_INVALID_ARG and wg == 0, kw
