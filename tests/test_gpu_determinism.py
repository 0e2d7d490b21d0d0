"""Every kernel class gives the same D bit for bit when a call is repeated,
on the default stream or a side stream: random N(0,1) · N(0,1/K) operands
(so any change in the order of the fp32 sums, or a race between waves or
workgroups, would show in the low bits), three calls per problem."""
import numpy as np
import pytest

import workloads
from gpu_util import run, run_mx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


FP_CASES = [
    ("f16", 4100, 8200, 192, "gemm_f16_256x256_w2x2_pers_dma"),
    ("f16", 4100, 4200, 200, "gemm_f16_256x256_w2x2_dma"),
    ("f16", 2100, 2000, 200, "gemm_f16_128x128_w2x2_ws_dma"),
    ("f16", 37, 16411, 200, "gemm_f16_64x128_w1x4_dma"),
    ("f16", 100, 16411, 200, "gemm_f16_128x128_w2x2_strip_dma"),
    ("f16", 200, 16400, 200, "gemm_f16_256x128_w2x2_dma"),
    ("f16", 64, 3584, 2048, "gemm_f16_64x32_w2x2_dma"),
    ("f16", 1000, 1000, 1000, "gemm_f16_64x64_w2x2_dma"),
    ("f16", 97, 131, 250, "gemm_f16_64x64_w2x2_scalar"),
    ("bf16", 4100, 8200, 192, "gemm_bf16_256x256_w2x2_pers_dma"),
]


@pytest.mark.parametrize("fmt,M,N,K,name", FP_CASES, ids=[c[4] for c in FP_CASES])
def test_repeated_calls_agree(fmt, M, N, K, name):
    plan = tg.tg_gemm_bf16_plan if fmt == "bf16" else tg.tg_gemm_f16_plan
    st, planned, _ = plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    assert st == tg.TG_OK and planned == name, planned
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((N, K)) / np.sqrt(K)
    if fmt == "bf16":
        a, b = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
    else:
        a, b = a.astype(np.float16), b.astype(np.float16)
    side = torch.cuda.Stream()
    outs = []
    for i, stream in enumerate((None, side, None)):
        d, _, st = run(a, b, M, N, K, stream=stream, label=f"determinism {name} call {i}", fmt=fmt)
        assert st == tg.TG_OK
        outs.append(np.asarray(d).view(np.uint16).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), name


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("M,N,K", [(2100, 2060, 512), (64, 16400, 1024)], ids=["256x256", "strip"])
def test_block_scaled_repeated_calls_agree(M, N, K, packed):
    qa, sa = workloads.random_mx(71 + M, M, K, 120, 126)
    qb, sb = workloads.random_mx(72 + N, N, K, 120, 126)
    outs = []
    for i in range(3):
        d, _, st = run_mx(qa, sa, qb, sb, M, N, K, label=f"determinism mx {M}x{N}x{K} call {i}", packed=packed)
        assert st == tg.TG_OK
        outs.append(np.asarray(d).view(np.uint16).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
