"""Seeded random problems through all three entry points against the oracle.

Every case draws its shape (three size classes, M and N up to 4400, K up to
600), leading dimensions, operand offsets and D's guard band from one seed:
mostly whole 16-byte rows (the direct-to-LDS path), sometimes odd K, odd
leading dimensions or misaligned pointers (the element-wise path).  These
complement the planner-coverage tests, which run every kernel
instantiation once; here the shapes and strides are arbitrary.  Half of
the fp16 and bf16 cases use {-1, 0, 1} operands, where D must equal the
oracle bit for bit; the others use N(0,1) data checked with the oracle's
tolerance on every element.  Operand padding holds NaN, and the guard band
around D must be untouched.  The block-scaled cases draw random codes and
scales (both scale layouts) with the element encoding of each operand drawn
too: E4M3 on both through tg_gemm_mxf8, otherwise E4M3 or E5M2 per operand
through tg_gemm_mx.  Each case prints its parameters before it runs."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SENTINEL, guard_intact, run, run_mx, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    size = rng.choice(["small", "mid", "large"], p=[0.45, 0.35, 0.2])
    hi = {"small": 400, "mid": 2300, "large": 4400}[size]
    M = int(rng.integers(1, hi))
    N = int(rng.integers(1, hi))
    # mostly whole 16-byte rows (the direct-to-LDS path), sometimes odd K
    K = int(8 * rng.integers(1, 75)) if rng.random() < 0.7 else int(rng.integers(1, 600))
    lda = K + int(rng.choice([0, 0, 0, 8, 64, 3]))
    ldb = K + int(rng.choice([0, 0, 0, 8, 128, 5]))
    a_off = int(rng.choice([0, 0, 0, 0, 0, 1]))
    b_off = int(rng.choice([0, 0, 0, 0, 0, 8]))
    guard = int(rng.integers(0, 3))
    exact = bool(rng.random() < 0.5)
    return rng, M, N, K, lda, ldb, a_off, b_off, guard, exact


def _operands(rng, M, N, K, lda, ldb, exact, fmt):
    if exact:
        a = rng.integers(-1, 2, size=(M, K)).astype(np.float64)
        b = rng.integers(-1, 2, size=(N, K)).astype(np.float64)
    else:
        a = rng.standard_normal((M, K))
        b = rng.standard_normal((N, K)) / np.sqrt(K)
    if fmt == "bf16":
        a, b = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
    else:
        a, b = a.astype(np.float16), b.astype(np.float16)
    return workloads.pad_columns(a, lda), workloads.pad_columns(b, ldb)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("seed", range(24))
def test_random_problem(seed, fmt):
    rng, M, N, K, lda, ldb, a_off, b_off, guard, exact = _draw(seed + (1000 if fmt == "bf16" else 0))
    if fmt == "bf16" and exact:
        K = min(K, 256)  # {-1, 0, 1} sums stay exact in bfloat16 up to K = 256
        lda, ldb = max(lda, K), max(ldb, K)
    a, b = _operands(rng, M, N, K, lda, ldb, exact, fmt)
    plan = tg.tg_gemm_bf16_plan if fmt == "bf16" else tg.tg_gemm_f16_plan
    st, name, _ = plan((1 << 20) + 2 * a_off, (1 << 20) + 2 * b_off, 1 << 20, M, N, K, lda, ldb, N + 2 * guard)
    assert st == tg.TG_OK
    label = f"random {fmt} seed={seed} {name} exact={exact}"
    d, full, st = run(a, b, M, N, K, guard=guard, a_off=a_off, b_off=b_off, label=label, fmt=fmt)
    assert st == tg.TG_OK
    assert guard_intact(full, M, N, guard), label
    res = oracle.gemm(a, b, M, N, K, fmt=fmt)
    if exact:
        bits = d if fmt == "bf16" else d.view(np.uint16)
        assert np.array_equal(bits, res.d.view(np.uint16)), label
    else:
        ok, worst, report = oracle.check(d, res)
        assert ok, f"{label}: {report}"


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("seed", range(8))
def test_random_block_scaled_problem(seed, packed):
    rng = np.random.default_rng(9500 + seed)
    big = rng.random() < 0.4
    M = int(rng.integers(1, 2300 if big else 300))
    N = int(rng.integers(1, 2300 if big else 300))
    K = 32 * int(rng.integers(1, 20))
    # element encodings from a stream of their own, so the shapes stay those
    # of E4M3 on both; E5M2 reaches 57344, so its scales sit lower (no sum
    # leaves binary16's range)
    fa, fb = (int(x) for x in np.random.default_rng(9800 + seed).integers(0, 2, size=2))
    fmts = ("e4m3", "e5m2")
    lo_hi = ((118, 124), (111, 115))
    qa, sa = workloads.random_mx(9600 + seed, M, K, *lo_hi[fa], fmt=fmts[fa])
    qb, sb = workloads.random_mx(9700 + seed, N, K, *lo_hi[fb], fmt=fmts[fb])
    nb = K // 32
    ld_s = max(4, (nb + 3) // 4 * 4) + 4 * int(rng.integers(0, 2))
    a = workloads.pad_bytes(qa, K + 16 * int(rng.integers(0, 3)))
    b = workloads.pad_bytes(qb, K + 16 * int(rng.integers(0, 3)))
    sa_p = workloads.pad_bytes(sa, ld_s, 0xff)
    sb_p = workloads.pad_bytes(sb, ld_s, 0xff)
    guard = int(rng.integers(0, 3))
    label = f"random block-scaled seed={seed} packed={packed} {M}x{N}x{K} formats=({fmts[fa]},{fmts[fb]})"
    res = oracle.gemm_mx(qa, sa, qb, sb, M, N, K, a_fmt=fmts[fa], b_fmt=fmts[fb])
    d, full, st = run_mx(a, sa_p, b, sb_p, M, N, K, guard=guard, label=label, packed=packed,
                         a_fmt=fa, b_fmt=fb)
    assert st == tg.TG_OK
    mask = np.ones(full.shape, bool)
    mask[guard:guard + M, guard:guard + N] = False
    assert bool(np.all(full[mask] == SENTINEL)), label
    ok, worst, report = oracle.check(d, res)
    assert ok, f"{label}: {report}"


def test_the_draws_reach_both_paths():
    """The fp16 draws above plan to the direct-to-LDS and the element-wise
    paths (checked on the host: the planner never touches memory)."""
    names = set()
    for seed in range(24):
        _, M, N, K, lda, ldb, a_off, b_off, guard, _ = _draw(seed)
        st, name, _ = tg.tg_gemm_f16_plan((1 << 20) + 2 * a_off, (1 << 20) + 2 * b_off, 1 << 20,
                                          M, N, K, lda, ldb, N + 2 * guard)
        names.add(name)
    say(f"random draws plan to: {sorted(names)}")
    assert any(n.endswith("_scalar") for n in names) and any(n.endswith("_dma") for n in names)
