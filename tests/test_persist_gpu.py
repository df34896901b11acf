"""Parity of the persistent-workgroup kernel (SPT_VARIANT_PERSIST) on an MI355X.

The persistent kernel walks a stream of 128 x 128 output tiles per
workgroup and writes each tile's C during the K-loop of the next one.  It
runs the same MFMAs in the same k order as the one-tile DIRECT kernel of the
same tile, so its C must be bit-identical to that kernel's ("Pipeline GPU
Kernel", Schritt 5: pipelining only reorders memory traffic) and within the
parity bar of the oracle.  Shapes cover one tile per workgroup, uneven
streams (some workgroups one tile more than others), every store window
(2, 4, 8 K tiles) with and without K tiles past the window, every ring
depth, and the low-K workload at full size.
"""
from __future__ import annotations

import numpy as np
import pytest

import software_pipelined_tiling_amd as spt
from software_pipelined_tiling_amd import inputs as I
from tests import parity
from tests.test_gemm_gpu import alloc_c, launch, operands, ref, run, sampled, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


def bk(dtype):
    return 64 // I.ELT_BYTES[dtype]


def ktiles_ok(kt, stages):
    return kt >= 2 and kt % 2 == 0 and (stages < 4 or kt >= 4)


# ---- full oracle parity, one or two tiles per workgroup ---------------------------
@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
def test_persist_matches_oracle(oracle_mod, dtype, b_col):
    """M = 384, N = 512 (12 tiles, one per workgroup) and K of 2, 6, 10 and 18 K
    tiles (window 2; window 4 plus 2 K tiles past it; 8 plus 2; 8 plus 10): full
    C against the oracle, every ring depth, and bit-identical to DIRECT."""
    M, N = 384, 512
    for kt in (2, 6, 10, 18):
        K = kt * bk(dtype)
        A, B = operands(dtype, b_col, M, N, K, 31 + kt)
        Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
        Cd = run(A, B, dtype, b_col, M, N, K, "direct", 3, 3)
        for s in (2, 3, 4):
            if not ktiles_ok(kt, s):
                continue
            C = run(A, B, dtype, b_col, M, N, K, "persist", s)
            parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)
            assert np.array_equal(C.view(np.uint32), Cd.view(np.uint32)), (dtype, b_col, kt, s)


# ---- streams of several tiles per workgroup, bit-identical to DIRECT ---------------
def both(A, B, dtype, b_col, M, N, K, stages):
    """C of DIRECT (tile 128 x 128, 3 stages) and of PERSIST with `stages`, on device."""
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    out = []
    for v, s in (("direct", 3), ("persist", stages)):
        print(f"[gpu] {dtype} {'col' if b_col else 'row'} M={M} N={N} K={K} {v}/{s}", flush=True)
        C = alloc_c(M, N + 4, dtype)
        launch(dA, dB, C, dtype, M, N, K, A.shape[1], B.shape[1], b_col, v, s, 3)
        out.append(C)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("M,N,kt", [(2176, 4096, 2), (4096, 2560, 4), (1280, 8192, 6), (2048, 4096, 16)])
def test_persist_streams_bit_identical(dtype, b_col, M, N, kt):
    """544, 640, 640 and 512 tiles over 512 workgroups (uneven streams of 1-2
    tiles, and one tile each); K of 2, 4, 6 and 16 K tiles.  Every ring depth
    gives C bit-identical to DIRECT, the padding columns untouched."""
    K = kt * bk(dtype)
    A, B = operands(dtype, b_col, M, N, K, 41 + kt, pad_nan=False)
    for s in (2, 3, 4):
        if not ktiles_ok(kt, s):
            continue
        Cd, Cp = both(A, B, dtype, b_col, M, N, K, s)
        assert torch.equal(Cd.view(torch.int32), Cp.view(torch.int32)), (dtype, b_col, M, N, kt, s)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("kt", [2, 4, 8, 12, 20])
def test_persist_long_streams_bit_identical(dtype, kt):
    """8192 x 8192: 4096 tiles, eight per workgroup (four output tiles per set of
    accumulators), every window, K tiles past the window for kt = 12 and 20."""
    M = N = 8192
    K = kt * bk(dtype)
    A, B = operands(dtype, False, M, N, K, 51 + kt, pad_nan=False)
    for s in (2, 3, 4):
        if not ktiles_ok(kt, s):
            continue
        Cd, Cp = both(A, B, dtype, False, M, N, K, s)
        assert torch.equal(Cd.view(torch.int32), Cp.view(torch.int32)), (dtype, kt, s)


# ---- the low-K workload at full size ---------------------------------------------
@pytest.mark.parametrize("K", I.LOWK_KS)
def test_full_bf16_lowk_persist(oracle_mod, K):
    """bf16 8192 x 8192 x K, K in {64, 128, 256, 512}: sampled outputs against the
    oracle (every output written)."""
    sampled(oracle_mod, I.w_bf16_lowk(K), "persist", 3)

