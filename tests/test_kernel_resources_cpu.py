"""Register and scratch budget of every gfx950 kernel, checked on the CPU.

The kernels keep their accumulators and operand fragments in registers; a
spill turns into scratch-memory traffic inside the K loop.  This compiles
the library's device code (the GEMM kernels and the measurement kernels) with the compiler's kernel-resource-usage remarks
(the same flags as the build) and requires, for every kernel in it: no
scratch memory, no spilled VGPRs or SGPRs, at most 256 VGPRs and 256 AGPRs
(one wave per SIMD with the whole register file), and an LDS size within
the 160 KiB of a compute unit."""
import re
import subprocess

import pytest

from dense_fp16_gemm_02_amd import build as B

pytestmark = pytest.mark.slow


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("ru")
    flags = [f for f in B.FLAGS if f != "-shared"]
    kernels = {}
    for i, src in enumerate(s for s in B.SOURCES if s.endswith(".hip")):
        cmd = [cc, *flags, f"-I{B.INCLUDE}", f"-I{B.CSRC}", "--cuda-device-only", "-c",
               src, "-o", str(tmp / f"dev{i}.o"), "-Rpass-analysis=kernel-resource-usage"]
        p = subprocess.run(cmd, capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-4000:]
        cur = None
        for line in p.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = kernels.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    return kernels


def test_every_kernel_reported(usage):
    names = " ".join(usage)
    for k in ("gemm_dma3_kernel", "gemm_dma_kernel", "gemm_vec_kernel", "gemm_mxf8_kernel",
              "gemm_mxf8_strip_kernel", "gemm_pers_kernel", "gemm_ws_kernel", "mfma_stream_kernel",
              "hbm_read_kernel"):
        assert k in names, k
    assert len(usage) >= 30


def test_no_scratch_no_spills(usage):
    bad = {}
    for name, r in usage.items():
        if (r.get("ScratchSize", 0) != 0 or r.get("VGPRs Spill", 0) != 0 or r.get("SGPRs Spill", 0) != 0
                or r.get("VGPRs", 0) > 256 or r.get("AGPRs", 0) > 256 or r.get("LDS Size", 0) > 160 * 1024):
            bad[name] = r
    assert not bad, bad
