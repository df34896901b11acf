"""Race detection on an MI355X: the rings built with SPT_POISON (libspt_poison.so).

In that build, after the barrier that frees a ring stage, every wave fills the
blocks its own copies are about to refill with NaN (fp16) or 127 (int8) and
waits for those writes before issuing the copies.  A read of a stage before
its copies have landed -- a missing or too-loose wait, a missing barrier, a
copy into a stage still being read -- then reaches C as NaN or as a wrong int8
sum.  Every ring (DIRECT with 2-4 stages on every tile, exact-fit and general;
PERSIST with 2-4 stages and every store window; the attention consumer's
DIRECT rings) must still match the oracle: fp16 within the tolerance, int8
bit for bit.
"""
from __future__ import annotations

import ctypes

import pytest

import software_pipelined_tiling_amd as spt
from tests import parity
from tests.test_gemm_gpu import alloc_c, operands, ref, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def plib(poison_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()
    L = ctypes.CDLL(poison_lib)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.spt_gemm_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp, i32, i32, i32, i32]
    L.spt_gemm_ex.restype = i32
    L.spt_attention.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, i32, vp, i32, i32]
    L.spt_attention.restype = i32
    L.spt_last_error.restype = ctypes.c_char_p
    return L


def poisoned(L, A, B, dtype, b_col, M, N, K, variant, stages, tile):
    print(f"[gpu] poison {dtype} {'col' if b_col else 'row'} {M}x{N}x{K} {variant}/{stages} tile={tile}", flush=True)
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    C = alloc_c(M, N, dtype)
    rc = L.spt_gemm_ex(M, N, K, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1], C.data_ptr(), N,
                       spt.DTYPE_CODES[dtype], torch.cuda.current_stream().cuda_stream, spt.COL if b_col else spt.ROW,
                       spt.VARIANT_CODES[variant], stages, tile)
    assert rc == 0, L.spt_last_error().decode()
    torch.cuda.synchronize()
    return C.cpu().numpy()


RINGS = [(1, 2), (1, 3), (1, 4), (2, 2), (2, 3), (3, 2), (3, 3), (3, 4), (4, 2), (4, 3), (5, 2), (5, 3), (5, 4),
         (6, 2)]


@pytest.mark.parametrize("dtype,b_col", [("f16", False), ("i8", True)])
@pytest.mark.parametrize("M,N,kt,tail", [(512, 512, 8, 0), (768, 1024, 14, 0), (300, 600, 7, 5), (300, 600, 7, 16)])
def test_direct_rings_never_read_a_stage_early(oracle_mod, plib, dtype, b_col, M, N, kt, tail):
    """Exact-fit shapes with an even number of K tiles, and ragged ones (general
    kernels) whose partial K tile goes through VGPRs (5 elements) or through the
    ring (16 elements, whole 16-byte chunks): every DIRECT ring of every tile
    matches the oracle."""
    K = kt * (64 if dtype == "i8" else 32) + tail
    A, B = operands(dtype, b_col, M, N, K, 91 + kt, pad_nan=False)
    Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
    for tile, s in RINGS:
        C = poisoned(plib, A, B, dtype, b_col, M, N, K, "direct", s, tile)
        parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)


@pytest.mark.parametrize("dtype,b_col", [("f16", False), ("i8", True)])
def test_persistent_rings_never_read_a_stage_early(oracle_mod, plib, dtype, b_col):
    """2048 x 1024 (128 tiles of 128 x 128 over the workgroups, some streams of
    two) with 2, 6 and 18 K tiles: every ring depth and store window."""
    M, N = 2048, 1024
    bk = 64 if dtype == "i8" else 32
    for kt in (2, 6, 18):
        K = kt * bk
        A, B = operands(dtype, b_col, M, N, K, 71 + kt, pad_nan=False)
        Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
        for s in (2, 3, 4):
            if s == 4 and kt < 4:
                continue
            C = poisoned(plib, A, B, dtype, b_col, M, N, K, "persist", s, 3)
            parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_rings_never_read_a_stage_early(oracle_mod, plib, dtype, D):
    """The attention consumer's DIRECT rings (2 and 3 stages) in the race-detection
    build: two slices of 300 queries against 700 keys (a ragged last key block)."""
    import numpy as np
    from software_pipelined_tiling_amd import inputs as I
    from tests.test_attention_gpu import dev
    Q, K, V = I.make_qkv(I.AttentionWorkload("t", 80 + D, 2, 300, 700, D, dtype))
    ref_o = oracle_mod.attention(Q, K, V, dtype, 1 / np.sqrt(D))
    dQ, dK, dV = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    for st in (2, 3):
        print(f"[gpu] poison attention {dtype} D={D} direct/{st}", flush=True)
        O = torch.full((2, 300, D), float("nan"), dtype=torch.float32, device="cuda")
        rc = plib.spt_attention(2, 300, 700, D, dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), O.data_ptr(),
                                1 / np.sqrt(D), spt.DTYPE_CODES[dtype], torch.cuda.current_stream().cuda_stream,
                                spt.VARIANT_DIRECT, st)
        assert rc == 0, plib.spt_last_error().decode()
        torch.cuda.synchronize()
        parity.check_attention(O.cpu().numpy(), ref_o, V, dtype)
