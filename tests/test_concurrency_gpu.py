"""Concurrent calls and captured launches of the GEMM and the attention
consumer, on an MI355X.

Between calls the library keeps only a thread-local error message, so calls
from several host threads, each on its own stream, must each give the output
of a single call.  A call is one kernel launch (two where a GEMM's last,
nearly empty round runs as a second grid) with no allocation, copy or memset,
so it can also be captured into a HIP graph: every replay must give the
output of an eager call on the inputs the buffers hold at that moment.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

import software_pipelined_tiling_amd as spt
from tests import parity
from tests.test_gemm_gpu import alloc_c, operands, ref, run, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


def test_threads_on_their_own_streams(oracle_mod):
    """Four host threads, eight calls each, on four streams into four outputs:
    every output bit-identical to one call's C, which matches the oracle."""
    M, N, K = 384, 512, 320
    A, B = operands("bf16", False, M, N, K, 61, pad_nan=False)
    expect = run(A, B, "bf16", False, M, N, K)
    parity.check_full(expect, ref(oracle_mod, A, B, "bf16", False, N, K), A, B, "bf16", False, M, N, K)
    dA, dB = to_dev(A, "bf16"), to_dev(B, "bf16")
    nthreads, reps = 4, 8
    outs = [alloc_c(M, N, "bf16") for _ in range(nthreads)]
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        for r in range(reps):
            rc = spt.spt_gemm_ex(M, N, K, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1], outs[i].data_ptr(),
                                 N, spt.BF16, streams[i].cuda_stream, spt.ROW, spt.VARIANT_AUTO, 0, 0)
            if rc != spt.SPT_OK:
                errors.append((i, r, spt.spt_status_string(rc), spt.spt_last_error()))

    print(f"[gpu] {nthreads} threads x {reps} calls, bf16 {M}x{N}x{K}", flush=True)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), expect.view(np.uint32))


def test_errors_stay_with_their_thread():
    """A refused call on one thread sets that thread's message only."""
    assert spt.spt_gemm(1, 1, 1, 0, 1, 0, 1, 0, 1, 9, 0) == spt.SPT_ERR_INVALID
    assert "dtype 9" in spt.spt_last_error()
    msgs = {}

    def bad():
        assert spt.spt_gemm(-1, 1, 1, 0, 1, 0, 1, 0, 1, spt.F16, 0) == spt.SPT_ERR_INVALID
        msgs["bad"] = spt.spt_last_error()

    t = threading.Thread(target=bad)
    t.start()
    t.join()
    assert "negative" in msgs["bad"]
    assert "dtype 9" in spt.spt_last_error()


@pytest.mark.parametrize("dtype,b_col,M,N,K", [("f16", False, 256, 384, 512), ("i8", True, 256, 384, 512),
                                               ("f16", False, 4224, 4000, 1040)],
                         ids=["f16", "i8_col", "f16_two_grids"])
def test_captured_in_a_hip_graph(oracle_mod, dtype, b_col, M, N, K):
    """One call captured into a graph, replayed six times over two operand sets
    that eager copies swap in between replays (C reset to a sentinel each time):
    every replay bit-identical to the eager call on the same operands.  The
    4224 x 4000 call is two launches (a grid, then a band of 128 x 128 tiles)."""
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW)
    assert rc == 0 and (pi.band_tile > 0) == (M == 4224)
    sets = [operands(dtype, b_col, M, N, K, 71 + i, pad_nan=False) for i in range(2)]
    eager = [run(A, B, dtype, b_col, M, N, K, ldc_pad=0) for A, B in sets]
    for (A, B), C in zip(sets, eager):
        parity.check_full(C, ref(oracle_mod, A, B, dtype, b_col, N, K), A, B, dtype, b_col, M, N, K)
    A0, B0 = sets[0]
    dA, dB = to_dev(A0, dtype), to_dev(B0, dtype)
    C = alloc_c(M, N, dtype)
    layout = "col" if b_col else "row"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a first call outside the capture
        spt.gemm(dA, dB, out=C, b_layout=layout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"[gpu] capture {dtype} {layout} {M}x{N}x{K}", flush=True)
    with torch.cuda.graph(g):
        spt.gemm(dA, dB, out=C, b_layout=layout)
    torch.cuda.synchronize()
    sentinel = alloc_c(M, N, dtype)
    for i in range(6):
        A, B = sets[i % 2]
        dA.copy_(to_dev(A, dtype))
        dB.copy_(to_dev(B, dtype))
        C.copy_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager[i % 2].view(np.uint32)), f"replay {i}"


def _attention_inputs(seed, dtype="f16", BH=3, Sq=300, Sk=333, D=128):
    from software_pipelined_tiling_amd import inputs as I
    from tests.test_attention_gpu import dev
    Q, K, V = I.make_qkv(I.AttentionWorkload("t", seed, BH, Sq, Sk, D, dtype))
    return (Q, K, V), tuple(dev(x, dtype) for x in (Q, K, V))


@pytest.mark.parametrize("variant,stages", [("direct", 2), ("reg", 2)])
def test_attention_captured_in_a_hip_graph(oracle_mod, variant, stages):
    """One attention call captured into a graph, replayed six times over two input
    sets that eager copies swap in between replays (O reset to NaN each time):
    every replay bit-identical to the eager call on the same inputs, which matches
    the oracle."""
    sets = [_attention_inputs(81 + i) for i in range(2)]
    eager = []
    for (Q, K, V), (dQ, dK, dV) in sets:
        O = spt.attention(dQ, dK, dV, variant=variant, stages=stages)
        torch.cuda.synchronize()
        eager.append(O.cpu().numpy())
        parity.check_attention(eager[-1], oracle_mod.attention(Q, K, V, "f16", 1 / np.sqrt(128)), V, "f16")
    dQ, dK, dV = (x.clone() for x in sets[0][1])
    O = torch.full(dQ.shape, float("nan"), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a first call outside the capture
        spt.attention(dQ, dK, dV, out=O, variant=variant, stages=stages)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"[gpu] capture attention {variant}/{stages}", flush=True)
    with torch.cuda.graph(g):
        spt.attention(dQ, dK, dV, out=O, variant=variant, stages=stages)
    torch.cuda.synchronize()
    sentinel = torch.full_like(O, float("nan"))
    for i in range(6):
        src = sets[i % 2][1]
        for d, s in zip((dQ, dK, dV), src):
            d.copy_(s)
        O.copy_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(O.cpu().numpy().view(np.uint32), eager[i % 2].view(np.uint32)), f"replay {i}"


def test_attention_threads_on_their_own_streams():
    """Four host threads, four attention calls each, on four streams into four
    outputs: every output bit-identical to one eager call's."""
    _, (dQ, dK, dV) = _attention_inputs(85, "bf16", BH=2, Sq=513, Sk=1000, D=64)
    expect = spt.attention(dQ, dK, dV)
    torch.cuda.synchronize()
    expect = expect.cpu().numpy()
    nthreads, reps = 4, 4
    outs = [torch.full(dQ.shape, float("nan"), dtype=torch.float32, device="cuda") for _ in range(nthreads)]
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        for r in range(reps):
            try:
                spt.attention(dQ, dK, dV, out=outs[i], stream=streams[i].cuda_stream)
            except Exception as e:  # noqa: BLE001 -- reported below
                errors.append((i, r, repr(e)))

    print(f"[gpu] {nthreads} threads x {reps} attention calls", flush=True)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), expect.view(np.uint32))
