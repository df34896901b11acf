"""Every (workload, variant, stages, tile) that bench.py times matches the
oracle over all of C (GPU).

bench.py times the headline workload (fp16 4096^3) under the library's choice
and over its sweep of every tile and (variant, stages) pair, and each side
workload (int8 4096^3 with column-major B, ragged bf16 4000 x 3000 x 1000,
fp16 256^3 with every pair on two tiles, bf16 8192^2 x K for the low-K
sweep) under the library's choice and as the unpipelined loop.  Here each of
those launches is compared with the oracle's full product on the same seeded
operands: int8 bit-exact, floats within the normalised tolerance, every
output written ("Pipeline GPU Kernel", Schritt 5: small sizes first, then the
target size).  One oracle product per workload is computed once and shared.
"""
from __future__ import annotations

import numpy as np
import pytest

import bench
import software_pipelined_tiling_amd as spt
from software_pipelined_tiling_amd import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


_cache: dict = {}


def workload(oracle_mod, w: I.Workload, with_ref: bool = True):
    """(A, B, device A, device B, oracle C or None) of `w`, computed once per module."""
    if w.name not in _cache or (with_ref and _cache[w.name][4] is None):
        _cache.clear()  # one full-size product held at a time
        A, B = I.make_operands(w)
        Cref = None
        if with_ref:
            print(f"[gpu] oracle {w.name}", flush=True)
            Cref = oracle_mod.gemm(A, B, w.dtype, b_col=w.b_col, K=w.K, N=w.N)
        _cache[w.name] = (A, B, bench.to_dev(A, w.dtype), bench.to_dev(B, w.dtype), Cref)
    return _cache[w.name]


def check(oracle_mod, w: I.Workload, variant="auto", stages=0, tile=0, K=None):
    K = w.K if K is None else K
    A, B, dA, dB, Cref = workload(oracle_mod, w, with_ref=K != 0)
    print(f"[gpu] {w.name} K={K} {variant}/{stages} tile={tile}", flush=True)
    if w.dtype == "i8":
        C = torch.full((w.M, w.N), 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    else:
        C = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device="cuda")
    rc = spt.spt_gemm_ex(w.M, w.N, K, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1], C.data_ptr(), w.N,
                         spt.DTYPE_CODES[w.dtype], torch.cuda.current_stream().cuda_stream,
                         spt.COL if w.b_col else spt.ROW, spt.VARIANT_CODES[variant], stages, tile)
    if rc == spt.SPT_ERR_UNSUPPORTED:
        return None  # not built (bench.py skips it too)
    assert rc == 0, spt.spt_last_error()
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    if K == 0:
        assert np.all(got == 0), "K = 0 must write zeros everywhere"
        return 0.0
    return parity.check_full(got, Cref, A, B, w.dtype, w.b_col, w.M, w.N, w.K)


def test_headline_auto(oracle_mod):
    check(oracle_mod, I.W_F16_4096)


@pytest.mark.parametrize("tile", bench.TILES)
@pytest.mark.parametrize("variant,stages", bench.PAIRS)
def test_headline_sweep(oracle_mod, tile, variant, stages):
    check(oracle_mod, I.W_F16_4096, variant, stages, tile)


SIDE = [I.W_I8_4096, I.W_BF16_RAGGED, I.W_F16_256] + [I.w_bf16_lowk(k) for k in I.LOWK_KS]


@pytest.mark.parametrize("w", SIDE, ids=lambda w: w.name.split(" (")[0].replace(" ", "_"))
def test_side_workload_auto_and_unpipelined(oracle_mod, w):
    check(oracle_mod, w)
    check(oracle_mod, w, "sync", 1)


@pytest.mark.parametrize("variant,stages", bench.PAIRS)
def test_small_case_every_pair(oracle_mod, variant, stages):
    """fp16 256^3 on the tile the library picks and on the pages' 128 x 256 tile."""
    rc, pp = spt.spt_plan(spt.F16, 256, 256, 256, spt.ROW)
    for tile in sorted({pp.tile_id, 1}):
        check(oracle_mod, I.W_F16_256, variant, stages, tile)


@pytest.mark.parametrize("K", I.LOWK_KS)
def test_low_k_store_only(oracle_mod, K):
    """The store-only launch bench.py times (the library's plan, run with K = 0)."""
    w = I.w_bf16_lowk(K)
    rc, pi = spt.spt_plan(spt.BF16, w.M, w.N, w.K, spt.ROW)
    assert rc == 0
    check(oracle_mod, w, {1: "sync", 2: "reg", 3: "direct"}[pi.variant], pi.stages, pi.tile_id, K=0)
