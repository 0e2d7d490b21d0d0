"""The stamping form of the persistent fp16 GEMM (tg_gemm_f16_xcd_stamps,
measurement only): D equals tg_gemm_f16's bit for bit (and the oracle's, on
small-integer operands), every workgroup writes a start no later than its
end and an XCD id below 8, the workgroups split evenly over the eight XCDs,
and no word past the workgroups' is written."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("dense_fp16_gemm_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    torch.cuda.init()


@pytest.mark.parametrize("M,N,K", [(4096, 8192, 128), (4100, 8200, 192)])
def test_stamped_call_matches_the_gemm(M, N, K):
    st, name, tiles = tg.tg_gemm_f16_plan(1 << 20, 1 << 20, 1 << 20, M, N, K, K, K, N)
    assert st == tg.TG_OK and name == "gemm_f16_256x256_w2x2_pers_dma", name
    a, b = workloads.small_int_pattern(M, N, K)
    A = torch.from_numpy(a).to("cuda:0")
    B = torch.from_numpy(b).to("cuda:0")
    D1 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
    D2 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
    _, cus, _, _ = tg.tg_device_info()
    room = 3 * cus + 64
    stamps = torch.full((room,), -1, dtype=torch.int64, device="cuda:0")
    say(f"xcd stamps {M}x{N}x{K}: {tiles} tiles, {cus} compute units")
    s = torch.cuda.current_stream()
    assert tg.tg_gemm_f16(A, B, D1, M, N, K, K, K, N, s) == tg.TG_OK
    st, wg = tg.tg_gemm_f16_xcd_stamps(A, B, D2, M, N, K, K, K, N, stamps, room, s)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    assert wg == min(cus // 8 * 8, tiles)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    res = oracle.gemm(a, b, M, N, K)
    assert np.array_equal(D2.cpu().numpy().view(np.uint16), res.d.view(np.uint16))
    w = stamps.cpu().numpy()
    assert np.all(w[3 * wg:] == -1)
    t = w[:3 * wg].reshape(wg, 3)
    assert np.all(t[:, 1] >= t[:, 0])
    assert np.all((t[:, 1] - t[:, 0]) < 100 * 10 ** 6)  # under a second on the 100 MHz clock
    xcc = t[:, 2]
    assert np.all((xcc >= 0) & (xcc < 8))
    counts = np.bincount(xcc, minlength=8)
    say(f"workgroups per XCD: {counts.tolist()}; workgroup w on XCD w mod 8: "
        f"{bool(np.all(xcc == np.arange(wg) % 8))}")
    assert np.all(counts == wg // 8)
