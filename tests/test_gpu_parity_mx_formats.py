"""The block-scaled GEMM with E5M2 elements (OCP MX's second FP8 encoding)
on one or both operands, through tg_gemm_mx and tg_gemm_mx_packed, against
the oracle: random codes of the whole encoding on both kernels and both
scale layouts (tolerance of the fp16 GEMM, every element), infinities and NaN
elements (IEEE propagation: infinity times zero is NaN), and a sum past
binary16's range rounding to infinity.  Each case prints its parameters
before it runs."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SENTINEL, run_mx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")

FMTS = ("e4m3", "e5m2")
COMBOS = [(1, 1), (1, 0), (0, 1)]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


def _scales(fmt_code, rng, rows, nb, ld):
    # E5M2 reaches 57344: scales 2^-14 .. 2^-12 keep its products small enough
    # that no sum leaves binary16's range
    lo, hi = (113, 115) if fmt_code else (120, 126)
    return workloads.pad_bytes(rng.integers(lo, hi + 1, size=(rows, nb)).astype(np.uint8), ld, 0xff)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("fa,fb", COMBOS)
@pytest.mark.parametrize("M,N,K", [(2100, 2060, 512), (64, 16400, 1024), (300, 200, 160)])
def test_random_codes(M, N, K, fa, fb, packed):
    rng = np.random.default_rng(M + N + K + 10 * fa + 20 * fb)
    a, _ = workloads.random_mx(int(rng.integers(1 << 30)), M, K, fmt=FMTS[fa])
    b, _ = workloads.random_mx(int(rng.integers(1 << 30)), N, K, fmt=FMTS[fb])
    nb = K // 32
    ld = max(4, (nb + 3) // 4 * 4)
    sa, sb = _scales(fa, rng, M, nb, ld), _scales(fb, rng, N, nb, ld)
    label = f"e5m2 random {M}x{N}x{K} formats=({FMTS[fa]},{FMTS[fb]}) packed={packed}"
    d, full, st = run_mx(a, sa, b, sb, M, N, K, guard=1, label=label, packed=packed, a_fmt=fa, b_fmt=fb)
    assert st == tg.TG_OK
    mask = np.ones(full.shape, bool)
    mask[1:1 + M, 1:1 + N] = False
    assert bool(np.all(full[mask] == SENTINEL)), label
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K, a_fmt=FMTS[fa], b_fmt=FMTS[fb])
    ok, worst, report = oracle.check(d, res)
    assert ok, f"{label}: {report}"


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("M,N", [(300, 200), (64, 16400)])
def test_infinities_and_nan(M, N, packed):
    """A +inf element of A against +1, 0 and -1 in B, a NaN element of B, and
    finite elements elsewhere: infinities, NaN and finite values land where
    the oracle puts them (NaN payloads are not compared)."""
    K = 96
    rng = np.random.default_rng(5 + M)
    a, _ = workloads.random_mx(11 + M, M, K, fmt="e5m2")
    b, _ = workloads.random_mx(12 + M, N, K, fmt="e5m2")
    a = np.where((a & 0x7c) > 0x50, a & np.uint8(0x83), a).astype(np.uint8)  # small finite values
    b = np.where((b & 0x7c) > 0x50, b & np.uint8(0x83), b).astype(np.uint8)
    a[3, 40] = 0x7c                                     # +inf in row 3 of A
    b[:, 40] = 0x3c                                     # +1 at that k ...
    b[1, 40], b[2, 40] = 0x00, 0xbc                     # ... but 0 and -1 in rows 1 and 2 of B
    b[7 % N, 70] = 0x7f                                 # a NaN element in row 7 of B
    nb = K // 32
    ld = 4
    sa = workloads.pad_bytes(np.full((M, nb), 127, np.uint8), ld, 0xff)
    sb = workloads.pad_bytes(np.full((N, nb), 127, np.uint8), ld, 0xff)
    d, _, st = run_mx(a, sa, b, sb, M, N, K, label=f"e5m2 inf/nan {M}x{N} packed={packed}", packed=packed,
                      a_fmt=1, b_fmt=1)
    assert st == tg.TG_OK
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K, a_fmt="e5m2", b_fmt="e5m2")
    got, want = d.astype(np.float64), res.d.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.isnan(want[3, 1]) and want[3, 0] == np.inf and want[3, 2] == -np.inf
    fin = ~np.isnan(want)
    assert np.array_equal(np.isinf(got[fin]), np.isinf(want[fin]))
    assert np.array_equal(got[np.isinf(want)], want[np.isinf(want)])
    ok, worst, report = oracle.check(np.where(np.isfinite(want), d, np.float16(0)),
                                     oracle.Result(np.where(np.isfinite(want), res.d, np.float16(0)),
                                                   np.where(np.isfinite(want), res.bound, 0.0),
                                                   np.where(np.isfinite(want), res.sum, 0.0),
                                                   res.rows, res.fmt))
    assert ok, report


def test_sum_past_binary16_range_is_infinity():
    M, N, K = 64, 16400, 32
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 0] = 0x7b                                      # 57344
    b[:, 0] = 0x40                                      # 2: 114688 > 65504
    b[5, 0] = 0x3c                                      # 1: 57344 stays finite
    s = workloads.pad_bytes(np.full((max(M, N), 1), 127, np.uint8), 4, 0xff)
    d, _, st = run_mx(a, s[:M], b, s[:N], M, N, K, label="e5m2 overflow", a_fmt=1, b_fmt=1)
    assert st == tg.TG_OK
    assert np.all(d[:, [0, 1, 6]] == np.inf) and np.all(d[:, 5] == 57344.0)


# E5M2 on both operands for every large workload; the mixed pair on the
# linear shape only (same kernel, other format fields)
LARGE_CASES = [(w, 1, 1) for w in workloads.WORKLOADS if w.M * w.N * w.K > 2 ** 31] + \
    [(workloads.BY_NAME["linear_8192x14336x4096"], 1, 0)]


@pytest.mark.parametrize("w,fa,fb", LARGE_CASES,
                         ids=lambda v: v.name if hasattr(v, "name") else FMTS[v])
def test_large_workloads_sampled_rows(w, fa, fb):
    """The benchmark's inputs and launch (packed scales, the kernel the plan
    picks) with E5M2 elements: the seeded draws encoded per block, D's
    sampled rows against the oracle on every column, the rest finite."""
    qa, sa, qb, sb = workloads.make_mx_inputs(w, FMTS[fa], FMTS[fb])
    rows = workloads.sample_rows(w)
    res = oracle.gemm_mx(qa, sa, qb, sb, w.M, w.N, w.K, rows=rows, a_fmt=FMTS[fa], b_fmt=FMTS[fb])
    label = f"{w.name} formats=({FMTS[fa]},{FMTS[fb]}) sampled rows"
    d, _, st = run_mx(qa, sa, qb, sb, w.M, w.N, w.K, label=label, packed=True, a_fmt=fa, b_fmt=fb)
    assert st == tg.TG_OK
    ok, worst, report = oracle.check(d[rows], res)
    assert ok, f"{label}: {report}"
    assert np.all(np.isfinite(d.astype(np.float32)))
