"""Pins for the E5M2 element encoding of the block-scaled oracle (OCP MX's
second FP8 encoding), each against something other than the oracle.

- E5M2 decode: all 256 codes against exact rational values derived here from
  the bit layout (sign, 5-bit exponent with bias 15, 2-bit fraction, exponent
  0 subnormal, exponent 31 infinity or NaN), against numpy's binary16 decode
  of the code as the upper byte of a binary16 pattern (E5M2 is exactly that
  byte), and the format's landmarks (largest finite 57344, smallest normal
  2^-14, smallest subnormal 2^-16).
- the GEMM with E5M2 on one or both operands: exact rational brute force on
  tiny shapes; at unit scales it equals the fp16 GEMM of the operands widened
  to binary16 by a byte shift (no decoder of the oracle involved);
  infinities and NaN follow IEEE arithmetic; sums past binary16's range
  round to infinity.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

INF = "inf"


def _frac_e5m2(code: int):
    sign = -1 if code & 0x80 else 1
    e, f = (code >> 2) & 31, code & 3
    if e == 31:
        return (INF, sign) if f == 0 else None
    if e == 0:
        return sign * Fraction(f, 4) * Fraction(1, 2 ** 14)
    return sign * (1 + Fraction(f, 4)) * Fraction(2) ** (e - 15)


def _frac_e4m3(code: int):
    sign = -1 if code & 0x80 else 1
    e, f = (code >> 3) & 15, code & 7
    if e == 0:
        return sign * Fraction(f, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)


def test_e5m2_decode_all_codes(oracle_lib):
    got = oracle.e5m2_to_double(np.arange(256, dtype=np.int64).astype(np.uint8))
    for c in range(256):
        want = _frac_e5m2(c)
        if want is None:
            assert np.isnan(got[c]), hex(c)
        elif isinstance(want, tuple):
            assert np.isinf(got[c]) and np.sign(got[c]) == want[1], hex(c)
        else:
            assert Fraction(got[c]) == want, hex(c)
    assert np.count_nonzero(np.isnan(got)) == 6 and np.count_nonzero(np.isinf(got)) == 2


def test_e5m2_is_the_upper_byte_of_binary16(oracle_lib):
    codes = np.arange(256, dtype=np.uint16)
    half = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    got = oracle.e5m2_to_double(codes.astype(np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(half))
    ok = ~np.isnan(half)
    assert np.array_equal(got[ok], half[ok])


def test_e5m2_landmarks(oracle_lib):
    v = oracle.e5m2_to_double(np.array([0x7b, 0x04, 0x01, 0x3c, 0xbc, 0x03, 0x7c, 0xfc], np.uint8))
    assert list(v[:6]) == [57344.0, 2.0 ** -14, 2.0 ** -16, 1.0, -1.0, 3 * 2.0 ** -16]
    assert v[6] == np.inf and v[7] == -np.inf


def _tame(codes):
    """E5M2 codes moved into exponents 10..20 (2^-5 .. 2^5 and their
    fractions), so that a short sum of their products is exact in float64
    (the full range spans 31 binades, more than a float64 significand)."""
    e = (codes >> 2) & 31
    return ((codes & 0x83) | (((10 + e % 11) & 31) << 2)).astype(np.uint8)


def _frac(fmt, code):
    return _frac_e5m2(code) if fmt == "e5m2" else _frac_e4m3(code)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("K", [1, 33, 96])
def test_brute_force_tiny_shapes(oracle_lib, fa, fb, K):
    M, N = 3, 2
    # scales 2^-4..2^-2 keep every sum below 65504 and (with the E5M2
    # exponents tamed below) exact in float64
    lo, hi, lo_b, hi_b = 123, 125, 123, 125
    a, sa = workloads.random_mx(700 + K, M, K, lo, hi, fmt=fa)
    b, sb = workloads.random_mx(800 + K, N, K, lo_b, hi_b, fmt=fb)
    if fa == "e5m2":
        a = _tame(a)
    if fb == "e5m2":
        b = _tame(b)
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K, a_fmt=fa, b_fmt=fb)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                x = _frac(fa, int(a[i, k])) * Fraction(2) ** (int(sa[i, k // 32]) - 127)
                y = _frac(fb, int(b[j, k])) * Fraction(2) ** (int(sb[j, k // 32]) - 127)
                s += x * y
            assert float(s) == s and abs(s) < 65504
            assert res.sum[i, j] == float(s)
            assert res.d[i, j] == np.float16(float(s))


def _widen(codes, fmt):
    """FP8 codes as binary16 values without the oracle: an E5M2 code is the
    upper byte of its binary16 pattern; E4M3 goes through the test's own
    rational decode (every E4M3 value is a binary16 value)."""
    if fmt == "e5m2":
        return (codes.astype(np.uint16) << 8).astype(np.uint16).view(np.float16)
    return np.vectorize(lambda c: np.float16(float(_frac_e4m3(int(c)))))(codes).astype(np.float16)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_unit_scales_reduce_to_the_fp16_gemm(oracle_lib, fa, fb):
    M, N, K = 9, 7, 160
    # magnitudes below 2^7 so that the fp16 GEMM's sums stay finite
    a, _ = workloads.random_mx(901, M, K, fmt=fa)
    b, _ = workloads.random_mx(902, N, K, fmt=fb)
    if fa == "e5m2":
        a = np.where((a & 0x7c) > 0x58, a & np.uint8(0x83), a).astype(np.uint8)
    if fb == "e5m2":
        b = np.where((b & 0x7c) > 0x58, b & np.uint8(0x83), b).astype(np.uint8)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    rm = oracle.gemm_mx(a, ones_a, b, ones_b, M, N, K, a_fmt=fa, b_fmt=fb)
    rf = oracle.gemm(_widen(a, fa), _widen(b, fb), M, N, K)
    assert np.array_equal(rm.d.view(np.uint16), rf.d.view(np.uint16))
    assert np.array_equal(rm.sum, rf.sum) and np.array_equal(rm.bound, rf.bound)


def test_infinities_and_nan(oracle_lib):
    """A single +inf element of A meets +1, 0 and -1 in three rows of B."""
    K = 32
    a = np.zeros((1, K), np.uint8)
    a[0, 3] = 0x7c                          # +inf
    b = np.zeros((3, K), np.uint8)
    b[0, 3], b[1, 3], b[2, 3] = 0x3c, 0x00, 0xbc   # +1, 0, -1
    b[:, 5] = 0x3c
    ones = np.full((3, 1), 127, np.uint8)
    res = oracle.gemm_mx(a, ones[:1], b, ones, 1, 3, K, a_fmt="e5m2", b_fmt="e5m2")
    d = res.d.astype(np.float64)[0]
    assert d[0] == np.inf and np.isnan(d[1]) and d[2] == -np.inf


def test_sum_past_binary16_range_rounds_to_infinity(oracle_lib):
    K = 32
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    a[0, 0], b[0, 0] = 0x7b, 0x40           # 57344 · 2 = 114688
    ones = np.full((1, 1), 127, np.uint8)
    res = oracle.gemm_mx(a, ones, b, ones, 1, 1, K, a_fmt="e5m2", b_fmt="e5m2")
    assert res.sum[0, 0] == 114688.0 and res.d[0, 0] == np.inf


def test_unknown_encoding_is_refused(oracle_lib):
    a = np.zeros((1, 32), np.uint8)
    s = np.full((1, 1), 127, np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_mx(a, s, a, s, 1, 1, 32, a_fmt="e3m4")


def test_e5m2_input_encoder(oracle_lib):
    """The input encoder (workloads, not the oracle) maps every finite E5M2
    value to its own code and keeps every element of a block within the
    encoding's relative spacing of the block's largest element."""
    vals = oracle.e5m2_to_double(np.arange(0x7c, dtype=np.uint8))
    assert np.array_equal(workloads.encode_e5m2(vals), np.arange(0x7c, dtype=np.uint8))
    assert np.array_equal(workloads.encode_e5m2(-vals[1:]), (np.arange(1, 0x7c) | 0x80).astype(np.uint8))
    x = np.random.default_rng(8).normal(size=(6, 100))
    codes, scales = workloads.mx_quantize(x, "e5m2")
    v = oracle.e5m2_to_double(codes) * np.repeat(oracle.e8m0_to_double(scales), 32, axis=1)[:, :100]
    amax = np.repeat(np.array([[np.abs(x[r, b:b + 32]).max() for b in range(0, 100, 32)] for r in range(6)]),
                     32, axis=1)[:, :100]
    assert np.all(np.abs(v - x) <= amax * 2.0 ** -2)
