"""The two measurement kernels do exactly the work their rates are computed
from (tg_mfma_ceiling, tg_hbm_read_ceiling through the C ABI).

With every operand element equal to one, each accumulator of the matrix-core
stream gains the instruction's K per MFMA it receives, so every lane's
output (the sum of its 256 accumulator values) is fixed by the instruction
count the flop figure assumes: 256·32·iters for the fp16 and bf16 forms
(64 MFMAs of K=32 per iteration over 64 accumulators, or 32 of K=16 in two
passes over 16), 256·64·iters for the block-scaled e4m3 form (16 MFMAs of
K=64, one pass).  Zero operands give zero.  The streaming read must touch
every 16-byte chunk exactly once: the XOR of all lanes' outputs equals the
XOR of every word of the buffer."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

tg = pytest.importorskip("dense_fp16_gemm_02_amd")
torch = pytest.importorskip("torch")

ONE = {"f16": 0x3C00, "bf16": 0x3F80}
E4M3_ONE = 0x38


@pytest.mark.parametrize("code,kind,per_iter", [
    ("TG_MFMA_F16_16X16X32", "f16", 256 * 32),
    ("TG_MFMA_F16_32X32X16", "f16", 256 * 32),
    ("TG_MFMA_BF16_16X16X32", "bf16", 256 * 32),
    ("TG_MFMA_MXF8_32X32X64", "e4m3", 256 * 64),
])
def test_mfma_stream_counts_its_instructions(code, kind, per_iter):
    dev = torch.device("cuda:0")
    if kind == "e4m3":
        ones = torch.full((4096,), E4M3_ONE, dtype=torch.uint8, device=dev)
        elems = ones.numel()
    else:
        ones = torch.full((2048,), ONE[kind], dtype=torch.int16, device=dev)
        elems = ones.numel()
    zeros = torch.zeros_like(ones)
    st, cus, _, _ = tg.tg_device_info()
    assert st == tg.TG_OK
    wg = min(cus, 64)
    out = torch.full((wg * 256,), -1.0, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for iters in (1, 3):
        say(f"mfma stream {code} iters={iters} ones")
        st = tg.tg_mfma_ceiling(getattr(tg, code), ones, elems, ones, elems, 1, iters, wg, out, stream)
        torch.cuda.synchronize()
        assert st == tg.TG_OK
        got = out.cpu().numpy()
        assert np.all(got == per_iter * iters), (code, iters, np.unique(got)[:8])
    say(f"mfma stream {code} zeros")
    st = tg.tg_mfma_ceiling(getattr(tg, code), zeros, elems, zeros, elems, 1, 2, wg, out, stream)
    torch.cuda.synchronize()
    assert st == tg.TG_OK and bool((out == 0).all())


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (4096 * 16 + 48, 7), ((64 << 20) + 16 * 1001, 2048)])
def test_hbm_read_touches_every_chunk_once(nbytes, wg):
    dev = torch.device("cuda:0")
    rng = np.random.Generator(np.random.PCG64(4242 + nbytes))
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    out = torch.full((wg * 256,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    say(f"hbm read {nbytes} bytes, {wg} workgroups")
    st = tg.tg_hbm_read_ceiling(buf, nbytes, wg, out, torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    assert st == tg.TG_OK
    folded = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert folded == np.bitwise_xor.reduce(words)
