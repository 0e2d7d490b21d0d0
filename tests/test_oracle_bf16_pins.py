"""Pins for the bfloat16 side of the CPU oracle, each against something other
than the oracle.

- bfloat16 decode: every one of the 65536 bit patterns against the float32
  whose upper half they are (numpy's own float32 decode).
- float64→bfloat16 rounding: every finite value, every midpoint between
  neighbours and the nearest float64 on either side of each midpoint, against
  a nearest-neighbour search over the table of representable values (ties to
  the even pattern); and, for float32 inputs, against the integer
  round-half-to-even on the float32 bit pattern.
- the GEMM: exact rational brute force on tiny shapes, all-ones closed forms
  with output rounding, an exact {-1, 0, 1} pattern, agreement with the fp16
  oracle's float64 sums on operands exact in both formats, and Σ|a||b|
  against a float64 library product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def _ref_decode(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_table():
    """Sorted non-negative finite bfloat16 values (bits 0..0x7f7f) plus the
    overflow point 2^128 standing for +inf (bits 0x7f80, an even pattern)."""
    bits = np.arange(0x7f80, dtype=np.uint16)
    vals = _ref_decode(bits)
    vals = np.append(vals, 2.0 ** 128)
    bits = np.append(bits, np.uint16(0x7f80))
    return vals, bits


_VALS, _BITS = _bf16_table()


def rne_by_search(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)
    a = np.abs(x)
    over = a >= 2.0 ** 128
    i = np.searchsorted(_VALS, a, side="right") - 1
    i = np.clip(i, 0, len(_VALS) - 2)
    lo, hi = _VALS[i], _VALS[i + 1]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_BITS[i] & 1).astype(bool))
    res = np.where(pick_hi, _BITS[i + 1], _BITS[i])
    res = np.where(a == lo, _BITS[i], res)
    res = np.where(over, np.uint16(0x7f80), res)
    return (res | sign).astype(np.uint16)


def test_decode_all_65536_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_double(bits)
    want = _ref_decode(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _probe_points():
    v = _VALS[:-1]
    mids = (v[:-1] + v[1:]) / 2.0          # exact in float64
    pts = np.concatenate([v, mids, np.nextafter(mids, 0.0), np.nextafter(mids, np.inf),
                          [2.0 ** 128, np.nextafter(2.0 ** 128, 0.0)]])
    return np.concatenate([pts, -pts])


def test_rounding_exhaustive_vs_search(oracle_lib):
    x = _probe_points()
    assert np.array_equal(oracle.double_to_bf16_bits(x), rne_by_search(x))


def test_rounding_float32_vs_integer_rne(oracle_lib):
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = raw.view(np.float32)
    f = f[np.isfinite(f)]
    u = f.view(np.uint32).astype(np.uint64)
    # round half to even on the dropped 16 bits (carry into the exponent is
    # the right behaviour, and reaches the infinity pattern on overflow)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = oracle.double_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_rounding_special_values(oracle_lib):
    x = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -2.0, 3.3895313892515355e38,
                  2.0 ** 128, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135])
    got = oracle.double_to_bf16_bits(x)
    want = [0x0000, 0x8000, 0x7f80, 0xff80, 0x3f80, 0xc000, 0x7f7f, 0x7f80, 0x0001, 0x0000, 0x0001]
    assert [int(g) for g in got] == want
    assert (int(oracle.double_to_bf16_bits(np.array([np.nan]))[0]) & 0x7fff) > 0x7f80
    # the largest finite value plus half its ulp is a tie with an odd
    # pattern (0x7f7f): it rounds up to infinity; just below it stays finite
    top, half = _ref_decode(np.array([0x7f7f]))[0], 2.0 ** (127 - 8)
    assert int(oracle.double_to_bf16_bits(np.array([top + half]))[0]) == 0x7f80
    assert int(oracle.double_to_bf16_bits(np.array([np.nextafter(top + half, 0)]))[0]) == 0x7f7f


def _frac_bf16(bits):
    v = _ref_decode(np.array([bits]))[0]
    return Fraction(v)


@pytest.mark.parametrize("K", [1, 2, 5, 13])
def test_brute_force_tiny_shapes(oracle_lib, K):
    M, N = 3, 4
    a = workloads.random_bf16(700 + K, (M, K))
    b = workloads.random_bf16(800 + K, (N, K))
    res = oracle.gemm(a, b, M, N, K, fmt="bf16")
    for i in range(M):
        for j in range(N):
            s = sum(_frac_bf16(a[i, k]) * _frac_bf16(b[j, k]) for k in range(K))
            want = rne_by_search(np.array([float(s)]))[0] if float(s) == s else None
            # s is exact in float64 for these sizes; the oracle rounds it once
            assert float(s) == s
            assert int(res.d[i, j]) == int(want)
            assert res.sum[i, j] == float(s)


@pytest.mark.parametrize("K,want", [(64, 64.0), (256, 256.0), (257, 256.0), (259, 260.0),
                                    (1000, 1000.0), (1001, 1000.0), (4097, 4096.0)])
def test_all_ones_rounds_the_sum(oracle_lib, K, want):
    """D = K exactly in float64; bfloat16 keeps 8 significant bits, so 257
    ties to 256 (even), 259 rounds up to 260 and 1001 down to 1000."""
    one = np.full((2, K), 0x3f80, dtype=np.uint16)
    res = oracle.gemm(one, one, 2, 2, K, fmt="bf16")
    assert np.all(res.sum == K)
    assert np.all(oracle.bf16_to_double(res.d) == want)


def test_small_int_pattern_exact(oracle_lib):
    M, N, K = 37, 29, 200
    a, b = workloads.small_int_pattern(M, N, K, "bf16")
    res = oracle.gemm(a, b, M, N, K, fmt="bf16")
    ai = (oracle.bf16_to_double(a)).astype(np.int64)
    bi = (oracle.bf16_to_double(b)).astype(np.int64)
    want = ai @ bi.T
    assert np.array_equal(oracle.bf16_to_double(res.d).astype(np.int64), want)


def test_agrees_with_fp16_oracle_on_shared_values(oracle_lib):
    """Operands exact in both formats give identical float64 sums."""
    M, N, K = 11, 13, 77
    af, bf = workloads.index_pattern(M, N, K)
    ab = workloads.to_bf16_bits(af.astype(np.float64))
    bb = workloads.to_bf16_bits(bf.astype(np.float64))
    r16 = oracle.gemm(af, bf, M, N, K)
    rbf = oracle.gemm(ab, bb, M, N, K, fmt="bf16")
    assert np.array_equal(r16.sum, rbf.sum)
    assert np.array_equal(r16.bound, rbf.bound)


def test_bound_and_sum_vs_float64_library(oracle_lib):
    M, N, K = 19, 23, 300
    a = workloads.random_bf16(901, (M, K))
    b = workloads.random_bf16(902, (N, K))
    res = oracle.gemm(a, b, M, N, K, fmt="bf16")
    A, B = _ref_decode(a), _ref_decode(b)
    assert np.allclose(res.sum, A @ B.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(res.bound, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)


def test_padding_is_never_read(oracle_lib):
    M, N, K = 5, 6, 40
    a = workloads.random_bf16(903, (M, K))
    b = workloads.random_bf16(904, (N, K))
    r0 = oracle.gemm(a, b, M, N, K, fmt="bf16")
    r1 = oracle.gemm(workloads.pad_columns(a, 48), workloads.pad_columns(b, 56), M, N, K, fmt="bf16")
    assert np.array_equal(r0.d, r1.d)


def test_check_uses_bf16_ulp(oracle_lib):
    M, N, K = 4, 4, 8
    a = workloads.random_bf16(905, (M, K))
    b = workloads.random_bf16(906, (N, K))
    res = oracle.gemm(a, b, M, N, K, fmt="bf16")
    ok, worst, _ = oracle.check(res.d.copy(), res)
    assert ok and worst == 0.0
    bad = res.d.copy()
    # move one element by 8·bound: far beyond the tolerance (4e-3·bound + ulp)
    bad[1, 2] = workloads.to_bf16_bits(np.array([oracle.bf16_to_double(res.d[1:2, 2])[0]
                                                 + 8 * res.bound[1, 2]]))[0]
    ok, worst, _ = oracle.check(bad, res)
    assert not ok
    assert oracle.ulp_bf16(np.array([1.0, 3.0, 2.0 ** -130]))[0] == 2.0 ** -7
    assert oracle.ulp_bf16(np.array([3.0]))[0] == 2.0 ** -6
    assert oracle.ulp_bf16(np.array([2.0 ** -130]))[0] == 2.0 ** -133
