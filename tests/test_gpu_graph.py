"""The entry points under stream capture: a call enqueues kernels only (no
allocation, no synchronization, no memset), so it can be recorded into a
HIP graph and replayed.  Each case captures one call on a side stream,
replays the graph several times with eager work and synchronizations
between the replays, and requires every replay's D to equal the eager
call's D bit for bit; the fp16 cases' operands are small integers, so D is
also compared with the oracle bit for bit, and the block-scaled case with
E5M2 and E4M3 operands is compared with the oracle within its tolerance."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import _bytes, pack_scales, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


def _replays_match(call, D, label, replays=4):
    """Eager call, then capture the same call and replay it; D is poisoned
    before every replay so a replay that writes nothing is caught."""
    stream = torch.cuda.Stream()
    say(f"graph {label}: eager")
    with torch.cuda.stream(stream):
        assert call(stream) == tg.TG_OK
    torch.cuda.synchronize()
    want = D.clone()
    g = torch.cuda.CUDAGraph()
    say(f"graph {label}: capture")
    with torch.cuda.graph(g, stream=stream):
        st = call(stream)
    assert st == tg.TG_OK
    for r in range(replays):
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph {label}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16), want.view(torch.int16)), f"{label}: replay {r} differs"
        junk = torch.randn(1 << 20, device="cuda:0").sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
    return want


@pytest.mark.parametrize("M,N,K,name", [(4096, 8192, 512, "gemm_f16_256x256_w2x2_pers_dma"),
                                        (2100, 2000, 200, "gemm_f16_128x128_w2x2_ws_dma"),
                                        (64, 16411, 200, "gemm_f16_64x128_w1x4_dma"),
                                        (64, 3584, 2048, "gemm_f16_64x32_w2x2_dma"),
                                        (97, 131, 250, "gemm_f16_64x64_w2x2_scalar")])
def test_fp16_call_replays_in_a_graph(M, N, K, name):
    st, planned, _ = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    assert st == tg.TG_OK and planned == name
    a, b = workloads.small_int_pattern(M, N, K)  # |D| <= K <= 2048: exact in binary16
    A = torch.from_numpy(a).to("cuda:0")
    B = torch.from_numpy(b).to("cuda:0")
    D = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    want = _replays_match(lambda s: tg.tg_gemm_f16(A, B, D, M, N, K, K, K, N, s), D, name)
    res = oracle.gemm(a, b, M, N, K)  # integer sums: exact, so bit for bit
    assert np.array_equal(want.cpu().numpy().view(np.uint16), res.d.view(np.uint16))


def test_block_scaled_packed_call_replays_in_a_graph():
    M, N, K = 2100, 2060, 512
    qa, sa = workloads.random_mx(61, M, K, 124, 130)
    qb, sb = workloads.random_mx(62, N, K, 124, 130)
    A, SA, B, SB = _bytes(qa), _bytes(sa), _bytes(qb), _bytes(sb)
    PA, PB = pack_scales(SA, M, K, sa.shape[1]), pack_scales(SB, N, K, sb.shape[1])
    D = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    want = _replays_match(lambda s: tg.tg_gemm_mxf8_packed(A, PA, B, PB, D, M, N, K, K, K, N, s), D,
                          "mxf8 packed")
    D2 = torch.empty_like(D)
    assert tg.tg_gemm_mxf8(A, SA, B, SB, D2, M, N, K, K, sa.shape[1], K, sb.shape[1], N,
                           torch.cuda.current_stream()) == tg.TG_OK
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), D2.view(torch.int16))


def test_block_scaled_mixed_encodings_replay_in_a_graph():
    # E5M2 elements in A, E4M3 in B, through tg_gemm_mx_packed; the E5M2
    # scales sit lower so that every sum stays inside binary16's range
    M, N, K = 2100, 2060, 512
    qa, sa = workloads.random_mx(63, M, K, 112, 115, fmt="e5m2")
    qb, sb = workloads.random_mx(64, N, K, 120, 126)
    A, SA, B, SB = _bytes(qa), _bytes(sa), _bytes(qb), _bytes(sb)
    PA, PB = pack_scales(SA, M, K, sa.shape[1]), pack_scales(SB, N, K, sb.shape[1])
    D = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    want = _replays_match(
        lambda s: tg.tg_gemm_mx_packed(A, PA, B, PB, D, M, N, K, K, K, N, tg.TG_MX_E5M2, tg.TG_MX_E4M3, s), D,
        "mx packed e5m2 x e4m3")
    D2 = torch.empty_like(D)
    assert tg.tg_gemm_mx(A, SA, B, SB, D2, M, N, K, K, sa.shape[1], K, sb.shape[1], N, tg.TG_MX_E5M2,
                         tg.TG_MX_E4M3, torch.cuda.current_stream()) == tg.TG_OK
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), D2.view(torch.int16))
    res = oracle.gemm_mx(qa, sa, qb, sb, M, N, K, a_fmt="e5m2", b_fmt="e4m3")
    ok, _, report = oracle.check(want.cpu().numpy(), res)
    assert ok, report
