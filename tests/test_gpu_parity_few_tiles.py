"""Problems with few output tiles: the 64×32 tiles (at most 128 tiles of
64×64 and K >= 2048: column shards of the skinny shape, small blocks with
deep K) and the 64×64 tiles with their 128-K tiles, including K that leaves
a partial last K-tile (K mod 128 = 8, 80, 120).  N(0,1) · N(0,1/K) data,
ragged M and N, D inside a guard band; every element against the oracle
within its tolerance, and the planner must pick the kernel named."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import guard_intact, run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


CASES = [
    ("f16", 64, 3584, 8192, "64x32_w2x2"),    # the skinny shape's 8-GPU column shard
    ("f16", 100, 1000, 2056, "64x32_w2x2"),   # partial last 128-K tile (8 of 128)
    ("f16", 37, 3000, 4104, "64x32_w2x2"),
    ("f16", 512, 512, 4096, "64x32_w2x2"),
    ("f16", 250, 700, 2048, "64x32_w2x2"),
    ("bf16", 64, 3584, 8192, "64x32_w2x2"),
    ("bf16", 100, 1000, 2056, "64x32_w2x2"),
    ("f16", 64, 3584, 2040, "64x64_w2x2"),    # K just short of the 64x32 rule; 120 of 128
    ("f16", 77, 333, 1104, "64x64_w2x2"),     # 80 of 128
    ("f16", 130, 200, 136, "64x64_w2x2"),     # one whole K-tile and 8 more
    ("bf16", 77, 333, 1104, "64x64_w2x2"),
]


@pytest.mark.parametrize("fmt,M,N,K,tile", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in CASES])
def test_few_tiles_random_data(fmt, M, N, K, tile):
    plan = tg.tg_gemm_bf16_plan if fmt == "bf16" else tg.tg_gemm_f16_plan
    st, name, _ = plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N + 2)
    assert st == tg.TG_OK and name == f"gemm_{fmt}_{tile}_dma", name
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((N, K)) / np.sqrt(K)
    if fmt == "bf16":
        a, b = workloads.to_bf16_bits(a), workloads.to_bf16_bits(b)
    else:
        a, b = a.astype(np.float16), b.astype(np.float16)
    label = f"few tiles {fmt} {M}x{N}x{K} {name}"
    d, full, st = run(a, b, M, N, K, guard=1, label=label, fmt=fmt)
    assert st == tg.TG_OK
    assert guard_intact(full, M, N, 1), label
    ok, worst, report = oracle.check(d, oracle.gemm(a, b, M, N, K, fmt=fmt))
    assert ok, f"{label}: {report}"
