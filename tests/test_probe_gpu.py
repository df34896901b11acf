"""bench.py's sustained-MFMA probe (libspt_probe.so, built from bench_probe.hip)
computes what it claims.

With every operand equal to one, each 16x16 MFMA adds k (32 for fp16/bf16,
64 for int8) to every accumulator element; the probe's per-lane checksum
adds two elements of each of its 64 accumulators, so after `iters` rounds it
is 64 * 2 * k * iters exactly.  The argument checks run before any HIP call
and are tested on the CPU.
"""
import ctypes
import os

import numpy as np
import pytest

from software_pipelined_tiling_amd import build as B

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(B.PROBE_LIB):
        B.build_probe()
    L = ctypes.CDLL(B.PROBE_LIB)
    L.spt_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.spt_probe_mfma.restype = ctypes.c_int
    return L


X0, Y0 = 1 << 32, 1 << 33


@pytest.mark.parametrize("args,status", [
    ((3, X0, 1024, 1, Y0), -1), ((0, 0, 1024, 1, Y0), -1), ((0, X0, 1024, 1, 0), -1), ((0, X0, 8, 1, Y0), -1),
    ((0, X0, 1024, -1, Y0), -1), ((0, X0 + 4, 1024, 1, Y0), -3),
])
def test_probe_validation(probe, args, status):
    assert probe.spt_probe_mfma(*args, None) == status


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,one,k", [(0, 0x3C00, 32), (1, 0x3F80, 32), (2, None, 64)])
@pytest.mark.parametrize("iters", [0, 1, 3])
def test_probe_checksum(probe, dtype, one, k, iters):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if dtype == 2:
        ops = torch.ones(4096, dtype=torch.int8, device="cuda")
    else:
        ops = torch.full((2048,), one, dtype=torch.int16, device="cuda")
    sink = torch.full((65536,), float("nan"), dtype=torch.float32, device="cuda")
    rc = probe.spt_probe_mfma(dtype, ops.data_ptr(), ops.numel() * ops.element_size(), iters, sink.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.all(sink.cpu().numpy() == 64 * 2 * k * iters)
