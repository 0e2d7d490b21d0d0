"""Every kernel instantiation the public entry points can launch, on the GPU.

For each name in ``planner_cases.CASES`` (fp16 and bf16: every tile × load
path) and ``planner_cases.MX_CASES`` / ``MXP_CASES`` (block-scaled FP8, row-major
and packed scales), one launch through
the C ABI whose plan must be that name, compared with the oracle on every
element and bit for bit: the operands are integer-valued (fp16: the index
pattern, |D| <= 6K, exact for K <= 341; bf16: values in {-1, 0, 1}, exact for
K <= 256; FP8: ±1 and 0 codes with per-block scales 2^-3..2^3, every partial
sum a multiple of 2^-6 that fp32 holds exactly), so any misplaced fragment,
swizzle, tile offset, tail mask or scale changes D.

Operand buffers are NaN-filled beyond the rows' K elements (and, for the
register path's huge row strides, across the gaps between rows), so a read
outside the operands' windows poisons D."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import NAN_BITS, SENTINEL, run_mx, say
from planner_cases import CASES, MX_CASES, MXF_CASES, MXP_CASES

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


def _strided_operand(x: np.ndarray, ld: int, offset: int, fmt: str):
    """Device buffer holding the rows of x (R × K, 16-bit) at row stride ld,
    starting `offset` elements past a 256-byte boundary; everything else is
    NaN.  Returns (buffer, pointer to element (0, 0))."""
    R, K = x.shape
    size = offset + (R - 1) * ld + K + 8 if R else 8
    buf = torch.full((size,), NAN_BITS[fmt], dtype=torch.int16, device="cuda:0")
    if R and K:
        raw = torch.from_numpy(np.ascontiguousarray(x).view(np.uint16).view(np.int16)).to("cuda:0")
        buf.as_strided((R, K), (ld, 1), offset).copy_(raw)
    return buf, buf.data_ptr() + 2 * offset


@pytest.mark.parametrize("name", sorted(CASES))
def test_instantiation_exact(name):
    fmt, c = CASES[name]
    M, N, K = c.M, c.N, c.K
    lda, ldb = c.lds()
    if fmt == "f16" and K <= 341:
        a, b = workloads.index_pattern(M, N, K)
    elif fmt == "f16":
        a, b = workloads.small_int_pattern(M, N, K)  # |D| <= K: exact in binary16
        assert K <= 2048
    else:
        # {-1, 0, 1}: every fp32 partial sum is an exact integer (|sum| <= K),
        # so D is the exact sum rounded once, here and in the oracle (exact in
        # bfloat16 itself for K <= 256)
        a, b = workloads.small_int_pattern(M, N, K, "bf16")
        assert K <= 4096
    A, a_ptr = _strided_operand(a, lda, c.a_off, fmt)
    B, b_ptr = _strided_operand(b, ldb, 0, fmt)
    D = torch.full((M * N + 8,), SENTINEL, dtype=torch.int16, device="cuda:0")
    plan = tg.tg_gemm_bf16_plan if fmt == "bf16" else tg.tg_gemm_f16_plan
    call = tg.tg_gemm_bf16 if fmt == "bf16" else tg.tg_gemm_f16
    st, planned, tiles = plan(a_ptr, b_ptr, D, M, N, K, lda, ldb, N)
    assert st == tg.TG_OK and planned == name, (planned, name)
    say(f"coverage {name}: M={M} N={N} K={K} lda={lda} ldb={ldb} a_off={c.a_off} tiles={tiles}")
    st = call(a_ptr, b_ptr, D, M, N, K, lda, ldb, N, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == tg.TG_OK
    d = D.cpu().numpy().view(np.uint16)
    assert np.all(d[M * N:] == SENTINEL)  # nothing written past the window
    d = d[:M * N].reshape(M, N)
    del A, B, D
    res = oracle.gemm(a, b, M, N, K, fmt=fmt)
    want = np.asarray(res.d).view(np.uint16)
    bad = np.argwhere(d != want)
    assert bad.size == 0, f"{name}: {len(bad)} elements differ, first at {tuple(bad[0])}"


ONE, MINUS_ONE, ZERO = 0x38, 0xb8, 0x00


@pytest.mark.parametrize("name", sorted(MX_CASES) + sorted(MXP_CASES))
def test_mx_instantiation_exact(name):
    packed = name in MXP_CASES
    c = MXP_CASES[name] if packed else MX_CASES[name]
    M, N, K = c.M, c.N, c.K
    rng = np.random.default_rng(K + M)
    codes = np.array([ONE, MINUS_ONE, ZERO], np.uint8)
    a = rng.choice(codes, size=(M, K))
    b = rng.choice(codes, size=(N, K))
    nb = K // 32
    ld = max(4, (nb + 3) // 4 * 4)
    sa = workloads.pad_bytes(rng.integers(124, 131, size=(M, nb)).astype(np.uint8), ld, 0xff)
    sb = workloads.pad_bytes(rng.integers(124, 131, size=(N, nb)).astype(np.uint8), ld, 0xff)
    if packed:
        st, planned, _ = tg.tg_gemm_mxf8_packed_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                                     M, N, K, K, K, N)
    else:
        st, planned, _ = tg.tg_gemm_mxf8_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                              M, N, K, K, ld, K, ld, N)
    assert st == tg.TG_OK and planned == name, (planned, name)
    d, _, st = run_mx(a, sa, b, sb, M, N, K, label=f"coverage {name}", packed=packed)
    assert st == tg.TG_OK
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    assert np.array_equal(d.view(np.uint16), res.d.view(np.uint16))


# +1, -1, 0 in each element encoding (E4M3, E5M2)
UNIT_CODES = {0: (0x38, 0xb8, 0x00), 1: (0x3c, 0xbc, 0x00)}


@pytest.mark.parametrize("name", sorted(MXF_CASES))
def test_mx_format_instantiation_exact(name):
    """Every instantiation of the other element encodings, on {-1, 0, 1}
    elements with random power-of-two scales: D equals the oracle bit for
    bit (every partial sum is exact in fp32)."""
    c, fa, fb, packed = MXF_CASES[name]
    M, N, K = c.M, c.N, c.K
    rng = np.random.default_rng(K + M + 7 * fa + 13 * fb)
    a = rng.choice(np.array(UNIT_CODES[fa], np.uint8), size=(M, K))
    b = rng.choice(np.array(UNIT_CODES[fb], np.uint8), size=(N, K))
    nb = K // 32
    ld = max(4, (nb + 3) // 4 * 4)
    sa = workloads.pad_bytes(rng.integers(124, 131, size=(M, nb)).astype(np.uint8), ld, 0xff)
    sb = workloads.pad_bytes(rng.integers(124, 131, size=(N, nb)).astype(np.uint8), ld, 0xff)
    if packed:
        st, planned, _ = tg.tg_gemm_mx_packed_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                                   M, N, K, K, K, N, fa, fb)
    else:
        st, planned, _ = tg.tg_gemm_mx_plan(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                            M, N, K, K, ld, K, ld, N, fa, fb)
    assert st == tg.TG_OK and planned == name, (planned, name)
    d, _, st = run_mx(a, sa, b, sb, M, N, K, label=f"coverage {name}", packed=packed, a_fmt=fa, b_fmt=fb)
    assert st == tg.TG_OK
    fmts = ("e4m3", "e5m2")
    res = oracle.gemm_mx(a, sa, b, sb, M, N, K, a_fmt=fmts[fa], b_fmt=fmts[fb])
    assert np.array_equal(d.view(np.uint16), res.d.view(np.uint16))
