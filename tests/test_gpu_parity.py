"""GPU parity: tg_gemm_f16 (through the C ABI) against the CPU oracle on the
same seeded inputs.

Acceptance per checked element: |D − ref| ≤ 4e-3·Σ|a||b| + ulp16(ref), D
finite.  The single-tile and ragged workloads are checked on every element;
the three large ones on 64 seeded rows plus the first and last row (every
column), in the launch configuration the benchmark times.  Integer-valued
operands make D exact, so those cases must match the oracle bit for bit,
which pins the MFMA fragment maps, the LDS swizzle and the tile offsets."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SENTINEL, guard_intact, run, say

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()  # raises if the HIP library is missing: no fallback
    torch.cuda.init()


def _check(d, res, what):
    ok, worst, report = oracle.check(d, res)
    assert ok, f"{what}: {report}"
    return worst


def _bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------------- workloads

@pytest.mark.parametrize("idx", [0, 1])
def test_workload_every_element(idx):
    w = workloads.WORKLOADS[idx]
    a, b = workloads.make_inputs(w)
    d, full, st = run(a, b, w.M, w.N, w.K, guard=8, label=w.name)
    assert st == tg.TG_OK
    assert guard_intact(full, w.M, w.N, 8)
    res = oracle.gemm(a, b, w.M, w.N, w.K)
    _check(d, res, w.name)


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_workload_sampled_rows(idx):
    """Full-size workloads, launched exactly as the benchmark launches them
    (tight leading dimensions, torch's current stream)."""
    w = workloads.WORKLOADS[idx]
    a, b = workloads.make_inputs(w)
    say(f"{w.name}: upload")
    A = torch.from_numpy(a).to("cuda:0")
    B = torch.from_numpy(b).to("cuda:0")
    D = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda:0")
    say(f"{w.name}: launch")
    st = tg.tg_gemm_f16(A, B, D, w.M, w.N, w.K, w.K, w.K, w.N, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == tg.TG_OK
    rows = workloads.sample_rows(w)
    d = D[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    res = oracle.gemm(a, b, w.M, w.N, w.K, rows=rows)
    _check(d, res, w.name)
    # the whole output is finite
    assert bool(torch.isfinite(D).all())


# ------------------------------------------------------ exact structure

@pytest.mark.parametrize("shape", [
    (128, 128, 64), (1000, 1000, 200), (257, 263, 336), (64, 520, 64), (1, 1, 64),
    (33, 1000, 336), (512, 512, 128), (300, 700, 72)])
def test_index_pattern_exact(shape):
    M, N, K = shape
    a, b = workloads.index_pattern(M, N, K)
    d, full, st = run(a, b, M, N, K, guard=3, label="index-pattern")
    assert st == tg.TG_OK and guard_intact(full, M, N, 3)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    res = oracle.gemm(a, b, M, N, K)
    assert np.array_equal(res.d.astype(np.int64), want)
    assert np.array_equal(_bits(d), _bits(res.d))


@pytest.mark.parametrize("M,N,K", [(300, 300, 64), (64, 64, 64), (520, 260, 128)])
def test_one_hot(M, N, K):
    """A[i,k] = [k == i mod K], B[j,k] = [k == (3j+1) mod K]: D[i,j] is 1
    exactly where the two indices meet, 0 elsewhere."""
    a = np.zeros((M, K), dtype=np.float16)
    b = np.zeros((N, K), dtype=np.float16)
    a[np.arange(M), np.arange(M) % K] = 1
    b[np.arange(N), (3 * np.arange(N) + 1) % K] = 1
    d, _, st = run(a, b, M, N, K, label="one-hot")
    assert st == tg.TG_OK
    want = ((np.arange(M) % K)[:, None] == ((3 * np.arange(N) + 1) % K)[None, :]).astype(np.float16)
    assert np.array_equal(_bits(d), _bits(want))


def test_rounding_is_nearest_even():
    """Rows whose fp32 sums sit on or next to binary16 rounding points; the
    sums are exact in fp32, so only the final conversion decides."""
    rows = [
        [1.0, 2.0 ** -11],                    # tie → 1.0 (even)
        [1.0, 2.0 ** -10, 2.0 ** -11],        # tie → 1 + 2^-9 (even)
        [1.0, 2.0 ** -11, 2.0 ** -12],        # above the tie → up (RTZ would give 1.0)
        [1.0, 2.0 ** -11, -(2.0 ** -13)],     # below the tie → down
        [-1.0, -(2.0 ** -11), -(2.0 ** -12)], # negative, above the tie in magnitude → away from 0
        [2048.0, 1.0],                        # tie at ulp 2 → 2048
        [2048.0, 1.0, 2.0],                   # 2051 → 2052
        [65504.0, 16.0],                      # 65520 rounds to +inf
        [65504.0, 8.0],                       # stays at 65504
        [0.5, 2.0 ** -12],                    # tie one binade down → 0.5
    ]
    K = 64
    a = np.zeros((len(rows), K), dtype=np.float16)
    for i, r in enumerate(rows):
        a[i, :len(r)] = r
    b = np.ones((32, K), dtype=np.float16)
    d, _, st = run(a, b, len(rows), 32, K, label="rounding")
    assert st == tg.TG_OK
    res = oracle.gemm(a, b, len(rows), 32, K)
    assert np.array_equal(_bits(d), _bits(res.d))
    assert _bits(d)[2, 0] == 0x3c01 and _bits(d)[7, 0] == 0x7c00 and _bits(d)[9, 0] == 0x3800


# ------------------------------------------- strides, alignment, tails

@pytest.mark.parametrize("case", [
    dict(M=200, N=136, K=96, lda=104, ldb=120, ldd=150),
    dict(M=77, N=301, K=40, lda=48, ldb=40, ldd=304),
    dict(M=256, N=256, K=64, lda=72, ldb=64, ldd=264),
])
def test_padded_strides_with_nan_poison(case):
    """Padding columns of A and B hold NaN: reading past K would poison D."""
    M, N, K = case["M"], case["N"], case["K"]
    a0 = workloads.random_f16(31, (M, K))
    b0 = workloads.random_f16(32, (N, K))
    a = workloads.pad_columns(a0, case["lda"])
    b = workloads.pad_columns(b0, case["ldb"])
    d, full, st = run(a, b, M, N, K, ldd=case["ldd"], label="padded")
    assert st == tg.TG_OK
    res = oracle.gemm(a0, b0, M, N, K)
    _check(d, res, "padded")
    # columns of D beyond N inside ldd stay untouched
    assert np.all(full[:M, N:case["ldd"]] == SENTINEL)


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 0), (0, 0, 1), (5, 7, 3)])
def test_misaligned_pointers(offs):
    M, N, K = 150, 190, 136
    a = workloads.random_f16(41, (M, K))
    b = workloads.random_f16(42, (N, K))
    d, full, st = run(a, b, M, N, K, guard=2, a_off=offs[0], b_off=offs[1], d_off=offs[2],
                      label="misaligned")
    assert st == tg.TG_OK and guard_intact(full, M, N, 2)
    _check(d, oracle.gemm(a, b, M, N, K), "misaligned")


@pytest.mark.parametrize("K", [1, 3, 7, 9, 63, 65, 77, 1001])
def test_k_not_multiple_of_8(K):
    M, N = 97, 131
    a = workloads.random_f16(50 + K, (M, K))
    b = workloads.random_f16(60 + K, (N, K))
    d, full, st = run(a, b, M, N, K, guard=1, label="odd-K")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    _check(d, oracle.gemm(a, b, M, N, K), f"K={K}")


@pytest.mark.parametrize("M", [1, 31, 64, 65, 255, 257])
@pytest.mark.parametrize("N", [1, 33, 128, 129, 511])
def test_ragged_tail_sweep(M, N):
    K = 200
    a = workloads.random_f16(70 + M, (M, K))
    b = workloads.random_f16(80 + N, (N, K))
    d, full, st = run(a, b, M, N, K, guard=4, label="tails")
    assert st == tg.TG_OK and guard_intact(full, M, N, 4)
    _check(d, oracle.gemm(a, b, M, N, K), f"{M}x{N}")


def test_large_tile_tails():
    """Shapes that take the largest tile with partial tiles in M, N and K."""
    M, N, K = 4100, 4200, 1000
    a = workloads.random_f16(91, (M, K))
    b = workloads.random_f16(92, (N, K))
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    say(f"large tails plan {name} tiles={tiles}")
    d, full, st = run(a, b, M, N, K, guard=2, label="large-tails")
    assert st == tg.TG_OK and guard_intact(full, M, N, 2)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(M - 300, M),
                                     workloads.sample_rows(workloads.Workload(9, "t", M, N, K, (), ()), 32)]))
    res = oracle.gemm(a, b, M, N, K, rows=rows)
    _check(d[rows], res, "large-tails")


@pytest.mark.parametrize("M,N,K,tile", [
    (64, 16411, 1000, "64x128_w1x4"),    # full strip, ragged N and K
    (37, 16400, 200, "64x128_w1x4"),     # ragged M; K spans 4 K-tiles (start offsets wrap)
    (1, 16385, 64, "64x128_w1x4"),       # one row; one K-tile
    (100, 16390, 776, "128x128_w2x2_strip"),
    (128, 16384, 1024, "128x128_w2x2_strip"),
    (200, 16500, 512, "256x128_w2x2"),
    (256, 16384, 264, "256x128_w2x2"),
])
def test_strip_tiles(M, N, K, tile):
    """Small M and large N take the column-strip tiles (one tile row covers
    M, each XCD starts at its own K offset); every element is checked."""
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N + 2)
    say(f"strip plan {name} tiles={tiles}")
    assert st0 == tg.TG_OK and name == f"gemm_f16_{tile}_dma"
    a = workloads.random_f16(300 + M, (M, K))
    b = workloads.random_f16(400 + K, (N, K))
    d, full, st = run(a, b, M, N, K, guard=1, label=f"strip {name}")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    _check(d, oracle.gemm(a, b, M, N, K), f"strip {M}x{N}x{K}")


def test_strip_index_pattern_exact():
    """Integer operands through the strip tile with K-offset rotation: exact."""
    M, N, K = 64, 16500, 328
    a, b = workloads.index_pattern(M, N, K)
    d, full, st = run(a, b, M, N, K, guard=2, label="strip index-pattern")
    assert st == tg.TG_OK and guard_intact(full, M, N, 2)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.astype(np.int64), want)


def test_second_wave_tiles_exact():
    """More 256×256 tiles than compute units (17×17 = 289), so some units run
    a second tile after the first.  Integer operands: every checked element
    is exact."""
    M, N, K = 4352 - 5, 4352 - 3, 136
    a, b = workloads.index_pattern(M, N, K)
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N + 2)
    say(f"second-wave plan {name} tiles={tiles}")
    assert name.startswith("gemm_f16_256x256_") and tiles == 289
    d, full, st = run(a, b, M, N, K, guard=1, label="second-wave exact")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(M - 300, M),
                                     np.arange(2048 - 8, 2048 + 8)]))
    want = a[rows].astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d[rows].astype(np.int64), want)


def test_second_wave_zero_k():
    """K = 0 through the 256×256 kernel with more tiles than compute units:
    every tile is +0 (its last K-tile runs unconditionally on stages that
    empty DMA ranges filled with zeros; the NaN operands are never read)."""
    M, N = 4352, 4352
    # lda = ldb = 8 keeps the direct-to-LDS kernel; the NaN columns are never read
    a = np.full((M, 8), np.nan, dtype=np.float16)
    b = np.full((N, 8), np.nan, dtype=np.float16)
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, 0, 8, 8, N + 2)
    say(f"second-wave K=0 plan {name} tiles={tiles}")
    assert name.endswith("_dma") and tiles == 289
    d, full, st = run(a, b, M, N, 0, guard=1, label="second-wave K=0")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    assert np.all(_bits(d) == 0)


def test_fewer_large_tiles_than_cus():
    """One GPU's share of the linear layer split by columns over eight GPUs,
    8192×1792×4096: 224 tiles of 256×256 on 256 CUs, which the largest tile
    takes from 160 tiles on; 66 sampled rows against the oracle."""
    M, N, K = 8192, 1792, 4096
    a = workloads.random_f16(93, (M, K))
    b = workloads.random_f16(94, (N, K), ("normal", 0.0, 1.0 / 64))
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    say(f"column-split plan {name} tiles={tiles}")
    assert name.startswith("gemm_f16_256x256_") and tiles == 224
    d, full, st = run(a, b, M, N, K, guard=1, label="column split")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    rows = workloads.sample_rows(workloads.Workload(8, "split", M, N, K, (), ()), 64)
    _check(d[rows], oracle.gemm(a, b, M, N, K, rows=rows), "column split")


@pytest.mark.parametrize("K", [8, 64, 72, 120])
def test_large_tile_short_k_exact(K):
    """Short K through the 256×256 kernel: one K-tile (K = 8, 64) or two whose
    first is the partial one (K = 72, 120); integer operands, exact."""
    M, N = 4096 + 40, 4096 + 24
    a, b = workloads.index_pattern(M, N, K)
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    say(f"short-K plan {name} tiles={tiles} K={K}")
    assert name.startswith("gemm_f16_256x256_") and name.endswith("_dma")
    d, full, st = run(a, b, M, N, K, guard=1, label=f"short-K {K}")
    assert st == tg.TG_OK and guard_intact(full, M, N, 1)
    rows = np.unique(np.concatenate([np.arange(0, 260), np.arange(M - 260, M)]))
    want = a[rows].astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d[rows].astype(np.int64), want)


def test_device_info():
    """tg_device_info reports the device the peak figures assume: gfx950, 256
    compute units, a maximum shader clock near 2.4 GHz."""
    st, cus, clk_khz, arch = tg.tg_device_info()
    say(f"device info: {arch} {cus} CUs {clk_khz} kHz")
    assert st == tg.TG_OK and arch.startswith("gfx950")
    assert cus == 256 and 2_000_000 <= clk_khz <= 3_000_000


# ------------------------------------------------------- degenerate cases

def test_zero_k_gives_positive_zero():
    M, N = 70, 90
    a = np.zeros((M, 0), dtype=np.float16)
    b = np.zeros((N, 0), dtype=np.float16)
    d, full, st = run(a, b, M, N, 0, guard=2, label="K=0")
    assert st == tg.TG_OK and guard_intact(full, M, N, 2)
    assert np.all(_bits(d) == 0)


def test_empty_m_or_n_touches_nothing():
    D = torch.full((16,), SENTINEL, dtype=torch.int16, device="cuda:0")
    A = torch.ones((4, 8), dtype=torch.float16, device="cuda:0")
    say("empty M/N")
    assert tg.tg_gemm_f16(A, A, D, 0, 4, 8, 8, 8, 4, None) == tg.TG_OK
    assert tg.tg_gemm_f16(A, A, D, 4, 0, 8, 8, 8, 1, None) == tg.TG_OK
    torch.cuda.synchronize()
    assert bool((D == SENTINEL).all())


def test_side_stream_and_determinism():
    w = workloads.WORKLOADS[1]
    a, b = workloads.make_inputs(w)
    s = torch.cuda.Stream()
    d1, _, st1 = run(a, b, w.M, w.N, w.K, stream=s, label="side-stream")
    d2, _, st2 = run(a, b, w.M, w.N, w.K, label="repeat")
    assert st1 == st2 == tg.TG_OK
    assert np.array_equal(_bits(d1), _bits(d2))


def test_torch_wrapper_matches():
    A = torch.randn(333, 256, device="cuda:0").half()
    B = torch.randn(444, 256, device="cuda:0").half()
    say("torch wrapper")
    D = tg.gemm(A, B)
    torch.cuda.synchronize()
    res = oracle.gemm(A.cpu().numpy(), B.cpu().numpy(), 333, 444, 256)
    _check(D.cpu().numpy(), res, "wrapper")


def test_torch_wrapper_refuses_overlapping_rows_and_mixed_devices():
    """A row stride below the row length (a stride-0 expand) would make the
    kernel read K·M elements from a K-element buffer: refused, not widened;
    so are operands on another device."""
    x = torch.randn(1, 64, device="cuda:0").half()
    B = torch.randn(32, 64, device="cuda:0").half()
    with pytest.raises(ValueError, match="row stride"):
        tg.gemm(x.expand(16, 64), B)
    with pytest.raises(ValueError, match="row stride"):
        tg.gemm(B, x.expand(16, 64))
    out = torch.empty(1, 16, device="cuda:0").half().expand(32, 16)
    with pytest.raises(ValueError, match="row stride"):
        tg.gemm(B, x.expand(16, 64).contiguous(), out=out)
    with pytest.raises(ValueError, match="GPU tensors"):
        tg.gemm(B, B.cpu())
    with pytest.raises(ValueError, match="device"):
        tg.gemm(B, B, out=torch.empty(32, 32, dtype=torch.float16))
    # a single row never uses its stride: an expanded one-row view is fine
    D = tg.gemm(x.expand(1, 64), B)
    torch.cuda.synchronize()
    res = oracle.gemm(x.cpu().numpy(), B.cpu().numpy(), 1, 32, 64)
    _check(D.cpu().numpy(), res, "one-row wrapper")


@pytest.mark.parametrize("K", [128, 192, 320])
def test_persistent_crosses_tile_boundaries_exact(K):
    """The persistent 256x256 kernel on 17 x 33 = 561 tiles: each of its 256
    workgroups takes two or three tiles, so its K-tile stream crosses tile
    boundaries (the next tile's first K-tiles load during the previous
    tile's last two; the epilogue is staged in the drained stages).  K spans
    2, 3 and 5 K-tiles; ragged M and N; D inside a guard band with an odd
    row stride (element-wise epilogue stores).  Integer operands: D must
    equal the oracle bit for bit, and nothing outside D's window changes."""
    M, N = 4100, 8200
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N + 6)
    assert st0 == tg.TG_OK and name == "gemm_f16_256x256_w2x2_pers_dma" and tiles == 561
    a, b = workloads.index_pattern(M, N, K)
    d, full, st = run(a, b, M, N, K, guard=3, label=f"persistent exact K={K}")
    assert st == tg.TG_OK and guard_intact(full, M, N, 3)
    res = oracle.gemm(a, b, M, N, K)
    assert np.array_equal(_bits(d), _bits(res.d))


def test_persistent_random_data_sampled():
    """Random N(0,1) and N(0,1/K) operands through the persistent kernel at a
    shape with a partial last wave (2 or 3 tiles per workgroup) and full
    K = 4096: sampled rows and every row of the last tile row, checked
    against the oracle's tolerance."""
    M, N, K = 4096 + 200, 8192 + 56, 4096
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    assert name == "gemm_f16_256x256_w2x2_pers_dma" and tiles == 17 * 33
    a = workloads.random_f16(5101, (M, K))
    b = workloads.random_f16(5102, (N, K), ("normal", 0.0, 1.0 / 64))
    say("persistent random: upload")
    A = torch.from_numpy(a).to("cuda:0")
    B = torch.from_numpy(b).to("cuda:0")
    D = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    st = tg.tg_gemm_f16(A, B, D, M, N, K, K, K, N, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == tg.TG_OK
    rows = np.unique(np.concatenate([workloads.sample_rows(workloads.Workload(9, "t", M, N, K, (), ()), 48),
                                     np.arange(4096, M)]))
    res = oracle.gemm(a, b, M, N, K, rows=rows)
    _check(D[torch.from_numpy(rows).to("cuda:0")].cpu().numpy(), res, "persistent random")
    assert bool(torch.isfinite(D).all())


@pytest.mark.parametrize("M,N,K", [(2100, 2000, 200), (2048, 4096, 328), (1537, 3001, 72), (3072, 3072, 64),
                                   (2048, 2048, 8), (1300, 2700, 136)])
def test_producer_consumer_tile_exact(M, N, K):
    """The producer/consumer 128x128 kernel (four waves only issue DMAs, four
    only multiply): K from 1 to 6 K-tiles with partial first K-tiles, ragged
    M and N, D inside a guard band with an odd row stride.  Integer operands:
    D equals the oracle bit for bit and nothing outside D's window changes."""
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N + 4)
    assert st0 == tg.TG_OK and name == "gemm_f16_128x128_w2x2_ws_dma"
    a, b = workloads.index_pattern(M, N, K)
    d, full, st = run(a, b, M, N, K, guard=2, label=f"producer/consumer exact {M}x{N}x{K}")
    assert st == tg.TG_OK and guard_intact(full, M, N, 2)
    res = oracle.gemm(a, b, M, N, K)
    assert np.array_equal(_bits(d), _bits(res.d))


def test_producer_consumer_tile_random_data():
    """Random N(0,1) and N(0,1/K) operands through the producer/consumer
    128x128 kernel at K = 4096, checked on sampled rows and the last tile row
    against the oracle's tolerance."""
    M, N, K = 2048 + 100, 4096 - 24, 4096
    st0, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    assert name == "gemm_f16_128x128_w2x2_ws_dma"
    a = workloads.random_f16(5201, (M, K))
    b = workloads.random_f16(5202, (N, K), ("normal", 0.0, 1.0 / 64))
    say("producer/consumer random: upload")
    A = torch.from_numpy(a).to("cuda:0")
    B = torch.from_numpy(b).to("cuda:0")
    D = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    st = tg.tg_gemm_f16(A, B, D, M, N, K, K, K, N, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == tg.TG_OK
    rows = np.unique(np.concatenate([workloads.sample_rows(workloads.Workload(9, "t", M, N, K, (), ()), 48),
                                     np.arange(2048, M)]))
    res = oracle.gemm(a, b, M, N, K, rows=rows)
    _check(D[torch.from_numpy(rows).to("cuda:0")].cpu().numpy(), res, "producer/consumer random")
    assert bool(torch.isfinite(D).all())
