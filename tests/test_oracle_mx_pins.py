"""Pins for the block-scaled FP8 side of the CPU oracle, each against
something other than the oracle.

- E4M3 decode: all 256 codes against exact rational values derived here from
  the bit layout (sign, 4-bit exponent with bias 7, 3-bit fraction, exponent 0
  subnormal, S.1111.111 NaN), plus the format's published landmarks (largest
  finite 448, smallest normal 2^-6, smallest subnormal 2^-9).
- UE8M0 decode: 2^(s-127) for every byte, NaN for 255.
- the GEMM: exact rational brute force on tiny shapes; unit scales reduce it
  to the fp16 GEMM of the decoded values (every E4M3 value is a binary16
  value); raising one block's scale by one doubles exactly that block's
  contribution (on either operand); closed forms; a partial last block; NaN
  propagation; padding never read.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def _frac_e4m3(code: int):
    sign = -1 if code & 0x80 else 1
    e, f = (code >> 3) & 15, code & 7
    if e == 15 and f == 7:
        return None  # NaN
    if e == 0:
        return sign * Fraction(f, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)


def test_e4m3_decode_all_codes(oracle_lib):
    got = oracle.e4m3_to_double(np.arange(256, dtype=np.int64).astype(np.uint8))
    for c in range(256):
        want = _frac_e4m3(c)
        if want is None:
            assert np.isnan(got[c]), hex(c)
        else:
            assert Fraction(got[c]) == want, hex(c)
    assert np.count_nonzero(np.isnan(got)) == 2


def test_e4m3_landmarks(oracle_lib):
    v = oracle.e4m3_to_double(np.array([0x7e, 0x08, 0x01, 0x38, 0xb8, 0x00, 0x80, 0x07], np.uint8))
    assert list(v[:5]) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert v[5] == 0.0 and v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == 7 * 2.0 ** -9  # largest subnormal


def test_e8m0_decode(oracle_lib):
    s = np.arange(256, dtype=np.int64).astype(np.uint8)
    v = oracle.e8m0_to_double(s)
    assert np.isnan(v[255])
    assert np.array_equal(v[:255], np.exp2(np.arange(255) - 127.0))


def _frac_gemm(a, sa, b, sb, M, N, K):
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                x = _frac_e4m3(int(a[i, k])) * Fraction(2) ** (int(sa[i, k // 32]) - 127)
                y = _frac_e4m3(int(b[j, k])) * Fraction(2) ** (int(sb[j, k // 32]) - 127)
                s += x * y
            out[i][j] = s
    return out


@pytest.mark.parametrize("K", [1, 31, 32, 33, 64, 96])
def test_brute_force_tiny_shapes(oracle_lib, K):
    M, N = 3, 2
    # scales 2^-4..2^-2 keep every sum below 65504 and exact in float64
    a, sa = workloads.random_mx(100 + K, M, K, 123, 125)
    b, sb = workloads.random_mx(200 + K, N, K, 123, 125)
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    exact = _frac_gemm(a, sa, b, sb, M, N, K)
    for i in range(M):
        for j in range(N):
            s = exact[i][j]
            assert float(s) == s and abs(s) < 65504
            assert res.sum[i, j] == float(s)
            assert res.d[i, j] == np.float16(float(s))  # numpy's float64 -> binary16 is RNE


def test_unit_scales_reduce_to_the_fp16_gemm(oracle_lib):
    M, N, K = 9, 7, 160
    a, _ = workloads.random_mx(301, M, K)
    b, _ = workloads.random_mx(302, N, K)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    rm = oracle.gemm_mx(a, ones_a, b, ones_b, M, N, K)
    af = oracle.e4m3_to_double(a).astype(np.float16)
    bf = oracle.e4m3_to_double(b).astype(np.float16)
    assert np.array_equal(af.astype(np.float64), oracle.e4m3_to_double(a))  # exact in fp16
    rf = oracle.gemm(af, bf, M, N, K)
    assert np.array_equal(rm.d.view(np.uint16), rf.d.view(np.uint16))
    assert np.array_equal(rm.sum, rf.sum) and np.array_equal(rm.bound, rf.bound)


@pytest.mark.parametrize("side", ["a", "b"])
def test_one_scale_step_doubles_one_block(oracle_lib, side):
    M, N, K = 4, 5, 96
    a, sa = workloads.random_mx(401, M, K, 126, 128)
    b, sb = workloads.random_mx(402, N, K, 126, 128)
    base = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    blk = 1
    if side == "a":
        sa2 = sa.copy(); sa2[2, blk] += 1
        bumped = oracle.gemm_mx(a, sa2, b, sb, M, N, K)
        part = oracle.gemm_mx(a[:, 32:64], sa[:, blk:blk + 1], b[:, 32:64], sb[:, blk:blk + 1], M, N, 32)
        want = base.sum.copy(); want[2, :] += part.sum[2, :]
    else:
        sb2 = sb.copy(); sb2[3, blk] += 1
        bumped = oracle.gemm_mx(a, sa, b, sb2, M, N, K)
        part = oracle.gemm_mx(a[:, 32:64], sa[:, blk:blk + 1], b[:, 32:64], sb[:, blk:blk + 1], M, N, 32)
        want = base.sum.copy(); want[:, 3] += part.sum[:, 3]
    assert np.array_equal(bumped.sum, want)
    changed = bumped.sum != base.sum
    assert changed.any()
    if side == "a":
        assert not changed[[0, 1, 3], :].any()
    else:
        assert not changed[:, [0, 1, 2, 4]].any()


@pytest.mark.parametrize("K,sa_byte,want", [(64, 127, 64.0), (2048, 127, 2048.0), (96, 128, 192.0),
                                            (100, 126, 50.0)])
def test_all_ones_closed_form(oracle_lib, K, sa_byte, want):
    one = np.full((2, K), 0x38, np.uint8)
    nb = (K + 31) // 32
    res = oracle.gemm_mx(one, np.full((2, nb), sa_byte, np.uint8), one, np.full((2, nb), 127, np.uint8), 2, 2, K)
    assert np.all(res.sum == want) and np.all(res.d == want)


def test_partial_last_block_uses_its_own_scale(oracle_lib):
    """K = 40: elements 32..39 form block 1 and take scale column 1 only."""
    K = 40
    a = np.full((1, K), 0x38, np.uint8)
    b = np.full((1, K), 0x38, np.uint8)
    sa = np.array([[127, 130]], np.uint8)     # block 1 scaled by 8
    sb = np.array([[127, 127]], np.uint8)
    res = oracle.gemm_mx(a, sa, b, sb, 1, 1, K)
    assert res.sum[0, 0] == 32 + 8 * 8


def test_nan_code_and_nan_scale_propagate(oracle_lib):
    M, N, K = 3, 3, 64
    a, sa = workloads.random_mx(501, M, K)
    b, sb = workloads.random_mx(502, N, K)
    a[1, 5] = 0x7f
    sb[2, 1] = 0xff
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    isn = np.isnan(res.d.astype(np.float64))
    assert isn[1, :].all() and isn[:, 2].all()
    assert not isn[0, 0] and not isn[0, 1] and not isn[2, 0]


def test_padding_is_never_read(oracle_lib):
    M, N, K = 5, 4, 72
    a, sa = workloads.random_mx(601, M, K)
    b, sb = workloads.random_mx(602, N, K)
    r0 = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    r1 = oracle.gemm_mx(workloads.pad_bytes(a, 96), workloads.pad_bytes(sa, 7, 0xff),
                        workloads.pad_bytes(b, 80), workloads.pad_bytes(sb, 5, 0xff), M, N, K)
    assert np.array_equal(r0.d.view(np.uint16), r1.d.view(np.uint16))


def test_quantizer_round_trip(oracle_lib):
    """The input encoder keeps every block within E4M3's relative spacing of
    its largest element (a sanity check of the test inputs, not of the
    oracle)."""
    x = np.random.default_rng(7).normal(size=(6, 100))
    codes, scales = workloads.mx_quantize(x)
    v = oracle.e4m3_to_double(codes) * np.repeat(oracle.e8m0_to_double(scales), 32, axis=1)[:, :100]
    amax = np.repeat(np.array([[np.abs(x[r, b:b + 32]).max() for b in range(0, 100, 32)] for r in range(6)]),
                     32, axis=1)[:, :100]
    # half of E4M3's relative step, or the clip of (448, 512) down to 448 at the top
    assert np.all(np.abs(v - x) <= amax * 2.0 ** -3)
    amax_b = np.array([[np.abs(x[r, b:b + 32]).max() for b in range(0, 100, 32)] for r in range(6)])
    assert np.array_equal(scales.astype(np.int64), np.floor(np.log2(amax_b)).astype(np.int64) - 8 + 127)
