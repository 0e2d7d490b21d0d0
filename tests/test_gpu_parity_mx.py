"""GPU parity of tg_gemm_mxf8 and tg_gemm_mxf8_packed (through the C ABI)
against the CPU oracle's block-scaled FP8 GEMM on the same seeded inputs
(the packed entry point with the scales converted on the device by
tg_mx_pack_scales; the tests marked with `packed` run both).

Acceptance per checked element: |D − ref| ≤ 4e-3·Σ_k|sa·a||sb·b| + ulp16(ref),
D finite; where every partial sum is exact in fp32 the comparison is
bit-exact.  Covered: the workloads whose K is whole 32-element blocks (small
ones on every element, the large ones on sampled rows; the ragged 1000³ case
runs at K = 992), exact operands that make every block's scale visible, a
partial last K-tile, tails in M and N with a guard band around D, padding of
operands and scale rows holding NaN codes, K = 0, and the layout errors."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SENTINEL, run_mx, say

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")

pytestmark = pytest.mark.gpu

ONE, MINUS_ONE, ZERO = 0x38, 0xb8, 0x00


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


def _guard_ok(full, M, N, g):
    mask = np.ones(full.shape, bool)
    mask[g:g + M, g:g + N] = False
    return bool(np.all(full[mask] == SENTINEL))


def _check(d, res, what):
    ok, worst, report = oracle.check(d, res)
    assert ok, f"{what}: {report}"


def _padded_scales(s, ld, fill=0xff):
    """Scale rows padded to ld bytes with NaN scale bytes (never to be used)."""
    return workloads.pad_bytes(s, ld, fill)


def _ld4(n):
    return max(4, (n + 3) // 4 * 4)


STRIP = "gemm_mxf8_64x128_w1x4_dma"
BIG = "gemm_mxf8_256x256_w2x2_g2_dma"    # scale words in pairs of K-tiles
BIG4 = "gemm_mxf8_256x256_w2x2_g4_dma"   # ... in groups of four (4 divides the K-tile count)


def _plan_name(M, N, K, lda, ldsa, ldb, ldsb, ldd, packed=False):
    """The row-major planner's kernel name, or the packed planner's with its
    `gemm_mxf8p_` prefix turned back into `gemm_mxf8_` (same kernels)."""
    if packed:
        st, name, tiles = tg.tg_gemm_mxf8_packed_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                                      M, N, K, lda, ldb, ldd)
        assert st == tg.TG_OK and name.startswith("gemm_mxf8p_")
        return name.replace("gemm_mxf8p_", "gemm_mxf8_")
    st, name, tiles = tg.tg_gemm_mxf8_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                           M, N, K, lda, ldsa, ldb, ldsb, ldd)
    assert st == tg.TG_OK
    return name


LAYOUTS = pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])


SMALL = [w for w in workloads.WORKLOADS if w.M * w.N * w.K <= 2 ** 31]


@LAYOUTS
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_workloads_every_element(w, packed):
    K = w.K - w.K % 32  # the ragged 1000³ case runs at K = 992
    qa, sa, qb, sb = workloads.make_mx_inputs(dataclasses.replace(w, K=K))
    res = oracle.gemm_mx(qa, sa, qb, sb, w.M, w.N, K)
    d, full, st = run_mx(qa, _padded_scales(sa, _ld4(K // 32)), qb, _padded_scales(sb, _ld4(K // 32)),
                         w.M, w.N, K, guard=3, label=w.name, packed=packed)
    assert st == tg.TG_OK
    _check(d, res, w.name)
    assert _guard_ok(full, w.M, w.N, 3)


@LAYOUTS
@pytest.mark.parametrize("w", [w for w in workloads.WORKLOADS if w.M * w.N * w.K > 2 ** 31], ids=lambda w: w.name)
def test_large_workloads_sampled_rows(w, packed):
    qa, sa, qb, sb = workloads.make_mx_inputs(w)
    rows = workloads.sample_rows(w)
    res = oracle.gemm_mx(qa, sa, qb, sb, w.M, w.N, w.K, rows=rows)
    d, _, st = run_mx(qa, sa, qb, sb, w.M, w.N, w.K, label=w.name, packed=packed)
    assert st == tg.TG_OK
    _check(d[rows], res, w.name)
    assert np.all(np.isfinite(d.astype(np.float32)))


def _pm1(seed, rows, K):
    rng = np.random.default_rng(seed)
    return rng.choice(np.array([ONE, MINUS_ONE, ZERO], np.uint8), size=(rows, K))


@pytest.mark.parametrize("M,N,K,kernel", [(256, 256, 128, STRIP), (300, 520, 256, STRIP), (77, 600, 1024, STRIP),
                                          (513, 129, 96, STRIP), (2100, 2050, 128, BIG), (2049, 2100, 96, BIG),
                                          (2100, 2050, 512, BIG4)])
@LAYOUTS
def test_unit_scales_exact(M, N, K, kernel, packed):
    """Values in {-1, 0, 1} with unit scales: D is an integer ≤ K, exact in
    fp32 and fp16, so every element must match the oracle bit for bit (on
    both kernels: 64×128 tiles for small problems, 256×256 for large)."""
    a, b = _pm1(11 + K, M, K), _pm1(12 + K, N, K)
    sa = np.full((M, _ld4(K // 32)), 127, np.uint8)
    sb = np.full((N, _ld4(K // 32)), 127, np.uint8)
    assert _plan_name(M, N, K, K, sa.shape[1], K, sb.shape[1], N + 4, packed) == kernel
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    d, full, st = run_mx(a, sa, b, sb, M, N, K, guard=2, label="unit scales", packed=packed)
    assert st == tg.TG_OK
    assert np.array_equal(d.view(np.uint16), res.d.view(np.uint16))
    assert _guard_ok(full, M, N, 2)


@pytest.mark.parametrize("M,N,K,kernel", [(256, 256, 256, STRIP), (190, 333, 384, STRIP), (260, 260, 96, STRIP),
                                          (2100, 2060, 256, BIG), (2070, 2090, 96, BIG),
                                          (2080, 2100, 1536, BIG4)])
@LAYOUTS
def test_random_scales_exact(M, N, K, kernel, packed):
    """Values ±1 and 0 with scales 2^-3..2^3 per block: every partial sum is a
    multiple of 2^-6 below 2^17 (K <= 1536), exact in fp32, so D is bit-exact.  A scale
    applied to the wrong block, lane half or operand changes D."""
    a, b = _pm1(21 + K, M, K), _pm1(22 + K, N, K)
    rng = np.random.default_rng(23 + K)
    nb = K // 32
    sa = _padded_scales(rng.integers(124, 131, size=(M, nb)).astype(np.uint8), _ld4(nb))
    sb = _padded_scales(rng.integers(124, 131, size=(N, nb)).astype(np.uint8), _ld4(nb))
    assert _plan_name(M, N, K, K, sa.shape[1], K, sb.shape[1], N, packed) == kernel
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    d, _, st = run_mx(a, sa, b, sb, M, N, K, label="random scales", packed=packed)
    assert st == tg.TG_OK
    assert np.array_equal(d.view(np.uint16), res.d.view(np.uint16))


@pytest.mark.parametrize("side", ["a", "b"])
@pytest.mark.parametrize("M,N", [(260, 270), (2100, 2060)])
@LAYOUTS
def test_each_block_scale_lands_on_its_block(side, M, N, packed):
    """All-ones operands with unit scales except one block of one row per
    probe: that row (column) of D gains exactly 7·32, nothing else moves
    (64×128 tiles at 260×270, 256×256 tiles at 2100×2060)."""
    K = 224   # two K-tiles, the second partial (blocks 4..6)
    nb = K // 32
    ones_a = np.full((M, K), ONE, np.uint8)
    ones_b = np.full((N, K), ONE, np.uint8)
    for probe, (row, blk) in enumerate([(0, 0), (1, 1), (33, 2), (31, 3), (64, 4), ((M if side == "a" else N) - 1, 6)]):
        sa = _padded_scales(np.full((M, nb), 127, np.uint8), 8)
        sb = _padded_scales(np.full((N, nb), 127, np.uint8), 8)
        (sa if side == "a" else sb)[row, blk] = 130
        d, _, st = run_mx(ones_a, sa, ones_b, sb, M, N, K, label=f"block probe {side} {row},{blk}", packed=packed)
        assert st == tg.TG_OK
        want = np.full((M, N), float(K))
        if side == "a":
            want[row, :] += 7 * 32
        else:
            want[:, row] += 7 * 32
        assert np.array_equal(d.astype(np.float64), want), f"probe {probe}: row {row} block {blk}"


@pytest.mark.parametrize("M,N,K", [(300, 280, 32), (300, 280, 96), (300, 280, 160), (300, 280, 4096 + 96),
                                   (2090, 2080, 32), (2090, 2080, 160), (2090, 2080, 1024 + 96)])
@LAYOUTS
def test_partial_k_tiles_and_nan_padding(M, N, K, packed):
    """K not a multiple of the 128-element stage: the missing elements are
    read as zero and their scale bytes (NaN here) are never applied; operand
    padding past K holds the NaN code (both kernels)."""
    # scales 2^-15..2^-9 keep |D| far below fp16's range for any codes
    qa, sa = workloads.random_mx(31 + K, M, K, 112, 118)
    qb, sb = workloads.random_mx(32 + K, N, K, 112, 118)
    nb = K // 32
    a = workloads.pad_bytes(qa, K + 48)
    b = workloads.pad_bytes(qb, K + 16 * 5)
    sa_p = _padded_scales(sa, _ld4(nb) + 4)
    sb_p = _padded_scales(sb, _ld4(nb))
    res = oracle.gemm_mx(qa, sa, qb, sb, M, N, K)
    d, full, st = run_mx(a, sa_p, b, sb_p, M, N, K, guard=2, label="partial K", packed=packed)
    assert st == tg.TG_OK
    _check(d, res, f"K={K}")
    assert _guard_ok(full, M, N, 2)


@pytest.mark.parametrize("M,N,K", [(64, 16400, 1024), (37, 16411, 224), (1, 16385, 32), (64, 16384, 4096 + 96)])
@LAYOUTS
def test_strip_every_element(M, N, K, packed):
    """Small M takes the column-strip kernel (each XCD starts at its own
    K-tile and wraps around); every element against the oracle, NaN scale
    bytes in the scale-row padding, a guard band around D."""
    qa, sa = workloads.random_mx(41 + K, M, K, 118, 124)
    qb, sb = workloads.random_mx(42 + K, N, K, 118, 124)
    nb = K // 32
    sa_p, sb_p = _padded_scales(sa, _ld4(nb) + 4), _padded_scales(sb, _ld4(nb))
    assert _plan_name(M, N, K, K, sa_p.shape[1], K, sb_p.shape[1], N + 4, packed) == STRIP
    res = oracle.gemm_mx(qa, sa, qb, sb, M, N, K)
    d, full, st = run_mx(qa, sa_p, qb, sb_p, M, N, K, guard=2, label="strip", packed=packed)
    assert st == tg.TG_OK
    _check(d, res, f"strip {M}x{N}x{K}")
    assert _guard_ok(full, M, N, 2)


@pytest.mark.parametrize("M,N,K", [(64, 16500, 384), (50, 16390, 96)])
@LAYOUTS
def test_strip_random_scales_exact(M, N, K, packed):
    """±1/0 operands with scales 2^-3..2^3 through the strip kernel: bit-exact."""
    a, b = _pm1(51 + K, M, K), _pm1(52 + K, N, K)
    rng = np.random.default_rng(53 + K)
    nb = K // 32
    sa = _padded_scales(rng.integers(124, 131, size=(M, nb)).astype(np.uint8), _ld4(nb))
    sb = _padded_scales(rng.integers(124, 131, size=(N, nb)).astype(np.uint8), _ld4(nb))
    assert _plan_name(M, N, K, K, sa.shape[1], K, sb.shape[1], N, packed) == STRIP
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    d, _, st = run_mx(a, sa, b, sb, M, N, K, label="strip random scales", packed=packed)
    assert st == tg.TG_OK
    assert np.array_equal(d.view(np.uint16), res.d.view(np.uint16))


@pytest.mark.parametrize("side", ["a", "b"])
@LAYOUTS
def test_strip_block_scale_lands_on_its_block(side, packed):
    """The block probes on the strip kernel: one block of one row raised to 2^3
    moves exactly that row (column) of D by 7·32."""
    M, N, K = 64, 16400, 224   # two K-tiles, the second partial
    nb = K // 32
    ones_a = np.full((M, K), ONE, np.uint8)
    ones_b = np.full((N, K), ONE, np.uint8)
    for probe, (row, blk) in enumerate([(0, 0), (33, 3), (63 if side == "a" else 16399, 6),
                                        (5, 4), (31 if side == "a" else 8191, 1)]):
        sa = _padded_scales(np.full((M, nb), 127, np.uint8), 8)
        sb = _padded_scales(np.full((N, nb), 127, np.uint8), 8)
        (sa if side == "a" else sb)[row, blk] = 130
        d, _, st = run_mx(ones_a, sa, ones_b, sb, M, N, K, label=f"strip block probe {side} {row},{blk}",
                          packed=packed)
        assert st == tg.TG_OK
        want = np.full((M, N), float(K))
        if side == "a":
            want[row, :] += 7 * 32
        else:
            want[:, row] += 7 * 32
        assert np.array_equal(d.astype(np.float64), want), f"probe {probe}: row {row} block {blk}"


@LAYOUTS
def test_strip_zero_k(packed):
    """K = 0 on the strip: every element +0 (no K-tile runs)."""
    M, N = 64, 16400
    a = np.zeros((M, 16), np.uint8)
    s = np.zeros((M, 4), np.uint8)
    b = np.zeros((N, 16), np.uint8)
    sb = np.zeros((N, 4), np.uint8)
    assert _plan_name(M, N, 0, 16, 4, 16, 4, N, packed) == STRIP
    d, full, st = run_mx(a, s, b, sb, M, N, 0, guard=1, label="strip K=0", packed=packed)
    assert st == tg.TG_OK and np.all(d == 0) and not np.signbit(d).any()
    assert _guard_ok(full, M, N, 1)


@LAYOUTS
def test_zero_k_and_empty(packed):
    a = np.zeros((5, 16), np.uint8)
    s = np.zeros((5, 4), np.uint8)
    d, full, st = run_mx(a, s, a, s, 5, 5, 0, guard=1, label="K=0", packed=packed)
    assert st == tg.TG_OK and np.all(d == 0) and not np.signbit(d).any()
    assert _guard_ok(full, 5, 5, 1)
    assert tg.tg_gemm_mxf8(0, 0, 0, 0, 0, 0, 5, 0, 32, 4, 32, 4, 5, None) == tg.TG_OK
    assert tg.tg_gemm_mxf8_packed(0, 0, 0, 0, 0, 0, 5, 0, 32, 32, 5, None) == tg.TG_OK


def test_layout_errors():
    a = torch.zeros(64 * 160, dtype=torch.uint8, device="cuda:0")
    s = torch.zeros(64 * 8, dtype=torch.uint8, device="cuda:0")
    d = torch.zeros(64 * 64, dtype=torch.float16, device="cuda:0")
    p, q, r = a.data_ptr(), s.data_ptr(), d.data_ptr()
    ok = (p, q, p, q, r, 64, 64, 128, 160, 4, 160, 4, 64, None)
    assert tg.tg_gemm_mxf8(*ok) == tg.TG_OK
    for bad in [dict(K=100, lda=160, ldb=160), dict(K=128, lda=136), dict(K=128, ldsa=5, ldsa_ok=False),
                dict(K=128, a_off=8), dict(K=128, s_off=2)]:
        args = list(ok)
        args[7] = bad.get("K", 128)
        args[8] = bad.get("lda", 160)
        args[9] = bad.get("ldsa", 4)
        args[0] = p + bad.get("a_off", 0)
        args[1] = q + bad.get("s_off", 0)
        say(f"mxf8 layout error {bad}")
        assert tg.tg_gemm_mxf8(*args) == tg.TG_ERR_LAYOUT, bad
    assert tg.tg_gemm_mxf8(p, q, p, q, r, 64, 64, 128, 100, 4, 160, 4, 64, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_mxf8(p, q, p, q, r, 64, 64, 128, 160, 2, 160, 4, 64, None) == tg.TG_ERR_INVALID_ARG
    torch.cuda.synchronize()


def _packed_reference(s, rows, K):
    """The packed layout written out from its definition in include/tg_gemm.h:
    byte of row r, block b at ((r/32)·G + b/16)·512 + (r%32)·16 + b%16 with G
    = ceil(K/512); 127 wherever r >= rows or b >= K/32."""
    nb, G = K // 32, (K + 511) // 512
    out = np.full(((rows + 31) // 32) * G * 512, 127, np.uint8)
    for r in range(rows):
        for b in range(nb):
            out[((r // 32) * G + b // 16) * 512 + (r % 32) * 16 + b % 16] = s[r, b]
    return out


@pytest.mark.parametrize("rows,K,lds", [(1, 32, 4), (100, 1568, 52), (64, 512, 16), (33, 4096, 128),
                                        (300, 96, 7)])
def test_pack_scales_layout(rows, K, lds):
    """tg_mx_pack_scales moves every byte of a row-major scale matrix (random
    bytes, padding of each row past K/32 set to 0xEE, never copied) to its
    place in the packed layout, and fills the rest with 127."""
    rng = np.random.default_rng(rows * 7 + K)
    s = rng.integers(0, 256, size=(rows, lds)).astype(np.uint8)
    s[:, K // 32:] = 0xEE
    from gpu_util import _bytes, pack_scales
    assert tg.tg_mx_packed_bytes(rows, K) == ((rows + 31) // 32) * ((K + 511) // 512) * 512
    say(f"pack scales rows={rows} K={K} lds={lds}")
    P = pack_scales(_bytes(s), rows, K, lds)
    torch.cuda.synchronize()
    got = P.cpu().numpy()[:tg.tg_mx_packed_bytes(rows, K)]
    assert np.array_equal(got, _packed_reference(s, rows, K))


@pytest.mark.parametrize("name", ["linear_8192x14336x4096", "square_4096x4096x4096", "skinny_64x28672x8192"])
def test_packed_bit_identical_full_size(name):
    """At the workloads' full sizes, in the benchmark's launch configuration:
    the packed entry point's D equals the row-major entry point's bit for
    bit (the same kernels, only the scale addressing differs; the row-major
    path is checked against the oracle above)."""
    w = workloads.BY_NAME[name]
    qa, sa, qb, sb = workloads.make_mx_inputs(w)
    from gpu_util import _bytes, pack_scales
    A, SA, B, SB = _bytes(qa), _bytes(sa), _bytes(qb), _bytes(sb)
    ldsa, ldsb = sa.shape[1], sb.shape[1]
    D0 = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda:0")
    D1 = torch.full((w.M, w.N), float("nan"), dtype=torch.float16, device="cuda:0")
    stream = torch.cuda.current_stream()
    say(f"packed vs row-major {name}")
    assert tg.tg_gemm_mxf8(A, SA, B, SB, D0, w.M, w.N, w.K, w.K, ldsa, w.K, ldsb, w.N, stream) == tg.TG_OK
    PA, PB = pack_scales(SA, w.M, w.K, ldsa), pack_scales(SB, w.N, w.K, ldsb)
    assert tg.tg_gemm_mxf8_packed(A, PA, B, PB, D1, w.M, w.N, w.K, w.K, w.K, w.N, stream) == tg.TG_OK
    torch.cuda.synchronize()
    assert torch.equal(D0.view(torch.int16), D1.view(torch.int16))


def test_packed_layout_errors():
    a = torch.zeros(64 * 160, dtype=torch.uint8, device="cuda:0")
    s = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    d = torch.zeros(64 * 64, dtype=torch.float16, device="cuda:0")
    p, q, r = a.data_ptr(), s.data_ptr(), d.data_ptr()
    ok = [p, q, p, q, r, 64, 64, 128, 160, 160, 64, None]
    assert tg.tg_gemm_mxf8_packed(*ok) == tg.TG_OK
    for i, v in [(7, 100), (8, 136), (1, q + 4), (3, q + 8), (0, p + 8)]:
        args = list(ok)
        args[i] = v
        if i == 7:
            args[8] = args[9] = 160
        say(f"mxf8 packed layout error arg {i}")
        assert tg.tg_gemm_mxf8_packed(*args) == tg.TG_ERR_LAYOUT, (i, v)
    assert tg.tg_mx_pack_scales(q, 64, 128, 4, q + 4, None) == tg.TG_ERR_LAYOUT
    torch.cuda.synchronize()
