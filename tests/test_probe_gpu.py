"""The sustained-MFMA measurement probe computes what it claims (GPU).

With every operand equal to one, each 16x16 MFMA adds k (32 for fp16/bf16,
64 for int8) to every accumulator element; the probe's per-lane checksum
adds two elements of each of its 64 accumulators, so after `iters` rounds it
is 64 * 2 * k * iters exactly.
"""
import numpy as np
import pytest

import software_pipelined_tiling_amd as spt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


@pytest.mark.parametrize("dtype,one,k", [(spt.F16, 0x3C00, 32), (spt.BF16, 0x3F80, 32), (spt.I8, None, 64)])
@pytest.mark.parametrize("iters", [0, 1, 3])
def test_probe_checksum(dtype, one, k, iters):
    if dtype == spt.I8:
        ops = torch.ones(4096, dtype=torch.int8, device="cuda")
    else:
        ops = torch.full((2048,), one, dtype=torch.int16, device="cuda")
    sink = torch.full((65536,), float("nan"), dtype=torch.float32, device="cuda")
    rc = spt.spt_probe_mfma(dtype, ops.data_ptr(), ops.numel() * ops.element_size(), iters, sink.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0, spt.spt_last_error()
    torch.cuda.synchronize()
    assert np.all(sink.cpu().numpy() == 64 * 2 * k * iters)
