"""Pins for the CPU oracle, each against something other than the oracle.

- binary16 decode: every one of the 65536 bit patterns against numpy's own
  float16 decode (an independent library routine).
- float64→binary16 rounding: every finite fp16 value, every midpoint between
  neighbours and the nearest float64 on either side of each midpoint, against
  a nearest-neighbour search over the table of representable values (ties to
  the even bit pattern) and against numpy's float64→float16 cast.
- the GEMM itself: exact rational brute force on tiny shapes (Python
  ``fractions``), constructed ties, closed forms (identity B, all-ones,
  rank-1, scaled-ones rows, K = 0), an integer index pattern against an exact
  int64 product, padded leading dimensions with NaN poison, and Σ|a||b|
  against a float64 library product.

A plausible slip in the oracle (a dropped or extra term, a wrong sign, a
transposed operand, lda/ldb mixed up, truncation or rounding through float32)
fails at least one of these.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


# ---------------------------------------------------------------- helpers

def _fp16_table():
    """Sorted non-negative finite binary16 values (bits 0..0x7bff) plus the
    overflow point 2^16 standing for +inf (bits 0x7c00, an even pattern)."""
    bits = np.arange(0x7c00, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    vals = np.append(vals, 65536.0)
    bits = np.append(bits, np.uint16(0x7c00))
    return vals, bits


_VALS, _BITS = _fp16_table()


def rne_by_search(x: np.ndarray) -> np.ndarray:
    """Round float64 → binary16 bits by nearest-neighbour search in the table
    of representable values; ties go to the even bit pattern."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)
    a = np.abs(x)
    out = np.empty(x.shape, dtype=np.uint16)
    over = a >= 65536.0
    i = np.searchsorted(_VALS, a, side="right") - 1
    i = np.clip(i, 0, len(_VALS) - 2)
    lo, hi = _VALS[i], _VALS[i + 1]
    dlo, dhi = a - lo, hi - a  # exact: lo <= a <= hi are close (Sterbenz)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_BITS[i] & 1).astype(bool))
    res = np.where(pick_hi, _BITS[i + 1], _BITS[i])
    res = np.where(a == lo, _BITS[i], res)
    res = np.where(over, np.uint16(0x7c00), res)
    out[...] = res | sign
    return out


def exact_rne_fraction(q: Fraction) -> int:
    """Exact binary16 rounding of a rational: nearest representable value,
    ties to the even pattern, values at or past 65520 to infinity."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a >= 65520:
        return sign | 0x7c00
    i = int(np.searchsorted(_VALS, float(a), side="right")) - 1
    # float(a) may round; step to the exact bracketing pair
    while i > 0 and Fraction(_VALS[i]) > a:
        i -= 1
    while Fraction(_VALS[i + 1]) <= a:
        i += 1
    lo, hi = Fraction(_VALS[i]), Fraction(_VALS[i + 1])
    if a == lo:
        return sign | int(_BITS[i])
    dlo, dhi = a - lo, hi - a
    if dhi < dlo or (dhi == dlo and int(_BITS[i]) & 1):
        return sign | int(_BITS[i + 1])
    return sign | int(_BITS[i])


def bits_of(x16: np.ndarray) -> np.ndarray:
    return np.asarray(x16, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------- binary16 decode

def test_decode_all_65536_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(mine[0x8000]) and not np.signbit(mine[0])


# ------------------------------------------------------ float64 → binary16

def _rounding_cases():
    vals = _VALS[:-1]                       # every finite non-negative fp16
    mids = (_VALS[:-1] + _VALS[1:]) / 2.0   # exact in float64 (12 bits)
    below = np.nextafter(mids, 0.0)
    above = np.nextafter(mids, np.inf)
    extra = np.array([0.0, 2.0 ** -25, 2.0 ** -26, 2.0 ** -24 * 0.75, 1e-300, 65504.0,
                      65519.999, 65520.0, 65535.0, 65536.0, 1e6, 1e300,
                      np.nextafter(2.0 ** -14, 0.0), 2.0 ** -14 - 2.0 ** -25])
    x = np.concatenate([vals, mids, below, above, extra])
    return np.concatenate([x, -x])


def test_rounding_exhaustive_vs_search(oracle_lib):
    x = _rounding_cases()
    mine = oracle.double_to_half_bits(x)
    ref = rne_by_search(x)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def test_rounding_exhaustive_vs_numpy(oracle_lib):
    x = _rounding_cases()
    mine = oracle.double_to_half_bits(x)
    ref = bits_of(x.astype(np.float16))
    assert np.array_equal(mine, ref)


def test_rounding_special_values(oracle_lib):
    f = oracle.double_to_half_bits
    assert f(np.array([np.inf]))[0] == 0x7c00
    assert f(np.array([-np.inf]))[0] == 0xfc00
    assert (f(np.array([np.nan]))[0] & 0x7c00) == 0x7c00 and (f(np.array([np.nan]))[0] & 0x3ff)
    assert f(np.array([-0.0]))[0] == 0x8000
    # ties: 1 + 2^-11 is halfway between 1 and 1+2^-10 → even (1.0)
    assert f(np.array([1.0 + 2.0 ** -11]))[0] == 0x3c00
    # 1 + 3·2^-11 is halfway between 1+2^-10 (odd) and 1+2^-9 (even)
    assert f(np.array([1.0 + 3 * 2.0 ** -11]))[0] == 0x3c02
    # double rounding through float32 would send this to 1.0 + 2^-10:
    # 1 + 2^-11 + 2^-40 is just above the tie, so RNE from float64 rounds up
    assert f(np.array([1.0 + 2.0 ** -11 + 2.0 ** -40]))[0] == 0x3c01
    # smallest subnormal and the tie below it
    assert f(np.array([2.0 ** -24]))[0] == 0x0001
    assert f(np.array([2.0 ** -25]))[0] == 0x0000
    assert f(np.array([3 * 2.0 ** -25]))[0] == 0x0002


# ------------------------------------------------------------ GEMM pins

def _tiny_operands(rng, M, N, K):
    """fp16 operands whose products and sums are exact in float64: A mixes
    ordinary values with subnormals and exact ties; B stays in [2^-4, 2^4]."""
    a = rng.standard_normal((M, K)) * 2.0
    sub = rng.random((M, K)) < 0.2
    a[sub] = rng.integers(-1023, 1024, size=int(sub.sum())) * 2.0 ** -24
    b = rng.choice([-1, 1], size=(N, K)) * np.exp2(rng.uniform(-4, 4, size=(N, K)))
    return a.astype(np.float16), b.astype(np.float16)


def _exact_gemm(a, b, M, N, K):
    fa = [[Fraction(float(a[i, k])) for k in range(K)] for i in range(M)]
    fb = [[Fraction(float(b[j, k])) for k in range(K)] for j in range(N)]
    return [[sum((fa[i][k] * fb[j][k] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


@pytest.mark.parametrize("K", [0, 1, 2, 3, 7, 16])
def test_brute_force_tiny_shapes(oracle_lib, K):
    rng = np.random.default_rng(77 + K)
    for M, N in itertools.product([1, 2, 3, 5], repeat=2):
        a, b = _tiny_operands(rng, M, N, K)
        res = oracle.gemm(a, b, M, N, K, nthreads=2)
        exact = _exact_gemm(a, b, M, N, K)
        for i in range(M):
            for j in range(N):
                # operands are chosen so that the float64 sum is exact
                assert Fraction(float(res.sum[i, j])) == exact[i][j]
                want = exact_rne_fraction(exact[i][j])
                got = int(bits_of(res.d[i:i + 1, j])[0])
                assert got == want, (M, N, K, i, j, exact[i][j])
                bnd = sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[j, k]))) for k in range(K))
                assert Fraction(float(res.bound[i, j])) == bnd


def test_constructed_ties(oracle_lib):
    # row sums that land exactly on binary16 midpoints, or just off them
    one = 1.0
    cases = [
        ([one, 2.0 ** -11], 0x3c00),                  # 1 + half ulp → 1 (even)
        ([one, 2.0 ** -10, 2.0 ** -11], 0x3c02),      # tie → even 1+2^-9
        ([one, 2.0 ** -11, 2.0 ** -24], 0x3c01),      # just above the tie → up
        ([one, 2.0 ** -11, -(2.0 ** -24)], 0x3c00),   # just below the tie → down
        ([2048.0, 1.0], 0x6800),                      # 2049 is a tie at ulp 2 → 2048
        ([2048.0, 1.0, 2.0], 0x6802),                 # 2051 tie → 2052
        ([65504.0, 16.0], 0x7c00),                    # 65520 rounds to +inf
        ([65504.0, 15.0], 0x7bff),
    ]
    for terms, want in cases:
        K = len(terms)
        a = np.array([terms], dtype=np.float16)
        assert np.array_equal(a.astype(np.float64)[0], np.array(terms))
        b = np.ones((1, K), dtype=np.float16)
        res = oracle.gemm(a, b, 1, 1, K)
        assert int(bits_of(res.d)[0, 0]) == want, terms


def test_identity_b(oracle_lib):
    M, K = 37, 50
    a = workloads.random_f16(5, (M, K))
    a[a == 0] = 1.0
    b = np.eye(K, dtype=np.float16)
    res = oracle.gemm(a, b, M, K, K)
    assert np.array_equal(bits_of(res.d), bits_of(a))


@pytest.mark.parametrize("K", [64, 1000, 2048, 4096, 8192])
def test_all_ones(oracle_lib, K):
    a = np.ones((3, K), dtype=np.float16)
    b = np.ones((4, K), dtype=np.float16)
    res = oracle.gemm(a, b, 3, 4, K)
    assert np.all(res.d.astype(np.float64) == K)
    assert np.all(res.bound == K)


def test_rank1_k1(oracle_lib):
    u = workloads.random_f16(11, (40, 1))
    v = workloads.random_f16(12, (33, 1))
    res = oracle.gemm(u, v, 40, 33, 1)
    want = (u.astype(np.float64) * v.astype(np.float64).T).astype(np.float16)
    assert np.array_equal(bits_of(res.d), bits_of(want))


def test_scaled_ones_rows(oracle_lib):
    K = 64
    av = workloads.random_f16(13, (9,))
    bv = workloads.random_f16(14, (7,))
    a = np.repeat(av[:, None], K, axis=1)
    b = np.repeat(bv[:, None], K, axis=1)
    res = oracle.gemm(a, b, 9, 7, K)
    want = (K * av.astype(np.float64)[:, None] * bv.astype(np.float64)[None, :]).astype(np.float16)
    assert np.array_equal(bits_of(res.d), bits_of(want))


def test_zero_k(oracle_lib):
    a = np.zeros((4, 0), dtype=np.float16)
    b = np.zeros((5, 0), dtype=np.float16)
    res = oracle.gemm(a, b, 4, 5, 0)
    assert np.all(bits_of(res.d) == 0)


def test_index_pattern_exact_with_padding(oracle_lib):
    M, N, K = 37, 29, 53
    a, b = workloads.index_pattern(M, N, K)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    res = oracle.gemm(a, b, M, N, K)
    assert np.array_equal(res.d.astype(np.int64), want)
    # padded leading dimensions filled with NaN must never be read
    ap = workloads.pad_columns(a, K + 11)
    bp = workloads.pad_columns(b, K + 5)
    res2 = oracle.gemm(ap, bp, M, N, K)
    assert np.array_equal(res2.d.astype(np.int64), want)


def test_bound_and_sum_vs_float64_library(oracle_lib):
    M, N, K = 48, 40, 1000
    a = workloads.random_f16(21, (M, K))
    b = workloads.random_f16(22, (N, K))
    res = oracle.gemm(a, b, M, N, K)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    bnd = np.abs(a64) @ np.abs(b64).T
    assert np.allclose(res.bound, bnd, rtol=1e-12, atol=0)
    s = a64 @ b64.T
    assert np.all(np.abs(res.sum - s) <= 1e-12 * bnd)


def test_row_subset_and_thread_count_agree(oracle_lib):
    w = workloads.WORKLOADS[1]
    a, b = workloads.make_inputs(w)
    M, N, K = 96, 80, w.K
    a, b = a[:M], b[:N]
    full = oracle.gemm(a, b, M, N, K, nthreads=1)
    rows = np.array([0, 5, 17, 95], dtype=np.int64)
    sub = oracle.gemm(a, b, M, N, K, rows=rows, nthreads=3)
    assert np.array_equal(bits_of(sub.d), bits_of(full.d[rows]))
    many = oracle.gemm(a, b, M, N, K, nthreads=7)
    assert np.array_equal(bits_of(many.d), bits_of(full.d))


def test_tolerance_catches_a_dropped_k_step(oracle_lib):
    """The acceptance inequality is tight enough that losing one 16-wide
    k-step (what a mis-indexed matrix-core step would do) is caught."""
    w = workloads.WORKLOADS[1]
    a, b = workloads.make_inputs(w)
    M = N = 128
    a, b = a[:M], b[:N]
    res = oracle.gemm(a, b, M, N, w.K)
    a2 = a.copy()
    a2[:, 32:48] = 0
    bad = oracle.gemm(a2, b, M, N, w.K)
    ok, worst, _ = oracle.check(bad.d, res)
    assert not ok and worst > 1.0
    ok, worst, _ = oracle.check(res.d, res)
    assert ok and worst == 0.0


def test_ulp16_definition():
    x = np.array([0.0, 2.0 ** -24, 2.0 ** -15, 2.0 ** -14, 1.0, 1.5, 2.0, 65504.0, -3.0])
    want = np.array([2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24, 2.0 ** -10, 2.0 ** -10,
                     2.0 ** -9, 32.0, 2.0 ** -9])
    assert np.array_equal(oracle.ulp16(x), want)
