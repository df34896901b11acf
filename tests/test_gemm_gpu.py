"""Parity of the HIP K-loop (through the C ABI) with the CPU oracle, on an MI355X.

Float results must be within the normalised tolerance of tests/parity.py;
int8 results must be bit-exact; closed forms and integer-valued inputs must
be bit-exact for every dtype; every (variant, stages) pair of one tile must
produce bit-identical C ("Pipeline GPU Kernel", Schritt 5: pipelining only
reorders the loads).  C is pre-filled with a sentinel so an unwritten output
or a write outside M x N shows up.
"""
from __future__ import annotations

import numpy as np
import pytest

import software_pipelined_tiling_amd as spt
from software_pipelined_tiling_amd import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PAIRS = [("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2), ("direct", 3), ("direct", 4)]
TILES = [1, 2, 3, 4, 5, 6]
SENT_F = np.uint32(0x7FC00ABC)   # a NaN payload no kernel produces
SENT_I = np.int32(0x7FFFFFFF)


def built(tile, variant, stages):
    """Rings of 64 KiB and 56 KiB stages (tiles 2, 4 and 6) hold two full stages at most
    in 160 KiB of LDS; the 256 x 256 x 128-byte tiles (2, 4) run 3 stages as 5
    half-stage slots."""
    if variant != "direct" or stages < 3:
        return True
    if tile in (2, 4):
        return stages == 3
    return tile != 6


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


def to_dev(x: np.ndarray, dtype: str):
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy())
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32).copy())
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int8).copy())
    return t.to("cuda")


def alloc_c(M, ldc, dtype):
    if dtype == "i8":
        return torch.full((M, ldc), int(SENT_I), dtype=torch.int32, device="cuda")
    return torch.full((M, ldc), int(SENT_F), dtype=torch.int32, device="cuda").view(torch.float32)


def launch(dA, dB, C, dtype, M, N, K, lda, ldb, b_col, variant="auto", stages=0, tile=0, stream=None):
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    rc = spt.spt_gemm_ex(M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, C.data_ptr(), C.shape[1],
                         spt.DTYPE_CODES[dtype], s, spt.COL if b_col else spt.ROW,
                         spt.VARIANT_CODES[variant], stages, tile)
    assert rc == 0, f"{spt.spt_status_string(rc)}: {spt.spt_last_error()}"


def run(A, B, dtype, b_col, M, N, K, variant="auto", stages=0, tile=0, ldc_pad=4):
    """Launch once; return the host copy of C[:, :N], checking the padding kept its sentinel."""
    print(f"[gpu] {dtype} {'col' if b_col else 'row'} M={M} N={N} K={K} lda={A.shape[1]} "
          f"ldb={B.shape[1]} {variant}/{stages} tile={tile}", flush=True)
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    ldc = -(-(N + ldc_pad) // 4) * 4  # 16-byte row pitch
    C = alloc_c(M, ldc, dtype)
    launch(dA, dB, C, dtype, M, N, K, A.shape[1], B.shape[1], b_col, variant, stages, tile)
    torch.cuda.synchronize()
    h = C.cpu().numpy()
    pad = h[:, N:].view(np.int32)
    want = SENT_I if dtype == "i8" else np.array(SENT_F).view(np.int32)
    assert np.all(pad == want), "write outside M x N"
    return np.ascontiguousarray(h[:, :N])


def operands(dtype, b_col, M, N, K, seed, lda_pad=0, ldb_pad=0, dist="uniform", lo=-1.0, hi=1.0,
             pad_nan=True):
    """Seeded operands with padded row pitches; padding holds NaN (int8: 127) so any
    leak of padding into the product is visible."""
    if dtype == "i8":
        lo, hi = -128, 127
    e = I.ELT_BYTES[dtype]
    q = 16 // e  # elements per 16 bytes: pitches stay 16-byte multiples
    lda = -(-(K + lda_pad) // q) * q if K else q
    bw = K if b_col else N
    ldb = -(-(bw + ldb_pad) // q) * q if bw else q
    w = I.Workload("t", seed, dtype, M, N, K, b_col, dist, lo, hi)
    a, b = I.make_operands(w, lda=lda, ldb=ldb)
    if pad_nan:
        fill = {"f16": 0x7E00, "bf16": 0x7FC0, "f32": np.nan, "i8": 127}[dtype]
        a[:, K:] = fill
        b[:, bw:] = fill
    return a, b


def ref(oracle_mod, A, B, dtype, b_col, N, K):
    return oracle_mod.gemm(A, B, dtype, b_col=b_col, K=K, N=N)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("tile", TILES)
def test_fp16_256_all_variants(oracle_mod, tile):
    """fp16 256^3, U[-1,1] (the small headline workload): every (variant, stages) pair
    matches the oracle and all of them are bit-identical."""
    w = I.W_F16_256
    A, B = I.make_operands(w)
    Cref = ref(oracle_mod, A, B, "f16", False, w.N, w.K)
    outs = {}
    for v, s in PAIRS:
        if not built(tile, v, s):
            continue
        outs[(v, s)] = run(A, B, "f16", False, w.M, w.N, w.K, v, s, tile)
        parity.check_full(outs[(v, s)], Cref, A, B, "f16", False, w.M, w.N, w.K)
    first = next(iter(outs.values()))
    for k, o in outs.items():
        assert np.array_equal(o.view(np.uint32), first.view(np.uint32)), f"{k} differs from {PAIRS[0]}"


SHAPES = [(1, 1, 1), (15, 17, 33), (17, 15, 8), (127, 129, 95), (129, 257, 161), (64, 64, 31),
          (64, 64, 33), (64, 64, 63), (64, 64, 65), (257, 300, 1000), (300, 520, 4)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
def test_ragged_shapes(oracle_mod, dtype, b_col):
    """Shapes that are not tile multiples, K tails of every width, padded pitches
    with NaN padding; default variant plus the unpipelined one."""
    for i, (M, N, K) in enumerate(SHAPES):
        A, B = operands(dtype, b_col, M, N, K, 100 + i, lda_pad=3, ldb_pad=5)
        Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
        for v, s in [("auto", 0), ("sync", 1)]:
            C = run(A, B, dtype, b_col, M, N, K, v, s)
            parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("tile", TILES)
def test_variants_bit_identical_ragged(oracle_mod, dtype, b_col, tile):
    """A ragged problem spanning several tiles in M, N and K: all variants agree
    with the oracle and with each other bit for bit."""
    M, N, K = 300, 600, 333 if dtype != "f32" else 300
    A, B = operands(dtype, b_col, M, N, K, 7, lda_pad=8, ldb_pad=8)
    Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
    outs = []
    for v, s in PAIRS:
        if not built(tile, v, s):
            continue
        C = run(A, B, dtype, b_col, M, N, K, v, s, tile)
        parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)
        outs.append(C)
    for C in outs[1:]:
        assert np.array_equal(C.view(np.uint32), outs[0].view(np.uint32))


RING_TAIL_TILES = {1: (2, 3, 4), 3: (2, 3, 4), 5: (2, 3, 4), 6: (2,)}  # DIRECT rings built per tile


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("tile", sorted(RING_TAIL_TILES))
def test_partial_tile_through_the_ring(oracle_mod, dtype, b_col, tile):
    """K tails of whole 16-byte chunks go through the DIRECT ring itself, zero-filled
    past K per chunk ("Hiding Memory Latency ...", section 8): with no full tile
    before them, inside the prologue, and after the steady state; NaN padding past K
    must not leak.  Every ring depth agrees with the oracle and bit for bit with the
    unpipelined loop, whose tail goes through VGPRs."""
    e = I.ELT_BYTES[dtype]
    BK = (128 if tile == 6 else 64) // e
    ch = 16 // e
    BM, BN = {1: (128, 256), 3: (128, 128), 5: (256, 256), 6: (256, 192)}[tile]
    M, N = BM + 37, BN + 20
    for K in (ch, BK + ch, 2 * BK + 3 * ch, 4 * BK + BK - ch, 9 * BK + 2 * ch):
        A, B = operands(dtype, b_col, M, N, K, 17 + K, lda_pad=8, ldb_pad=8)
        Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
        C1 = run(A, B, dtype, b_col, M, N, K, "sync", 1, tile)
        parity.check_full(C1, Cref, A, B, dtype, b_col, M, N, K)
        for st in RING_TAIL_TILES[tile]:
            rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW,
                                  spt.VARIANT_DIRECT, st, tile)
            assert rc == 0 and pi.tail_ring == 1 and pi.k_tail > 0
            C = run(A, B, dtype, b_col, M, N, K, "direct", st, tile)
            parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)
            assert np.array_equal(C.view(np.uint32), C1.view(np.uint32)), (tile, st, K)


HALF_RING_SHAPES = [(256, 256, 1), (512, 256, 2), (256, 512, 3), (512, 512, 4), (256, 768, 5), (768, 256, 8)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("tile", [2, 4])
def test_half_stage_ring(oracle_mod, dtype, b_col, tile):
    """The 3-stage ring of the 256 x 256 x 128-byte tiles runs as 5 half-stage slots (A
    and B of a K tile in separate slots, the copies of the next A kept in flight at
    every wait).  Exact-fit shapes with 1 to 8 K tiles (the prologue copies past the
    last tile are empty) and a ragged one with a K tail (general kernels): the results
    agree with the oracle and bit for bit with the 2-stage ring."""
    BK = 128 // I.ELT_BYTES[dtype]
    cases = [(M, N, kt * BK) for M, N, kt in HALF_RING_SHAPES] + [(300, 600, 3 * BK + 5)]
    for i, (M, N, K) in enumerate(cases):
        rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW,
                              spt.VARIANT_DIRECT, 3, tile)
        assert rc == 0 and pi.half_stage_slots == 5 and pi.lds_bytes == 5 * pi.a_stage_bytes
        A, B = operands(dtype, b_col, M, N, K, 40 + i, lda_pad=8, ldb_pad=8)
        Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
        C3 = run(A, B, dtype, b_col, M, N, K, "direct", 3, tile)
        parity.check_full(C3, Cref, A, B, dtype, b_col, M, N, K)
        C2 = run(A, B, dtype, b_col, M, N, K, "direct", 2, tile)
        assert np.array_equal(C3.view(np.uint32), C2.view(np.uint32)), (tile, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_integer_valued_bit_exact(oracle_mod, dtype):
    """Integer inputs (|a|,|b| <= 4; int8 full range): every partial sum is exact in the
    accumulator, so C equals the oracle bit for bit."""
    M, N, K = 384, 512, 1024
    lo, hi = (-4, 4) if dtype != "i8" else (-128, 127)
    w = I.Workload("int", 21, dtype, M, N, K, False, "intgrid", lo, hi)
    A, B = I.make_operands(w)
    Cref = ref(oracle_mod, A, B, dtype, False, N, K)
    for v, s in [("direct", 3), ("reg", 2), ("sync", 1)]:
        C = run(A, B, dtype, False, M, N, K, v, s)
        assert np.array_equal(C.astype(np.float64), Cref.astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "i8"])
@pytest.mark.parametrize("b_col", [False, True])
def test_identity_and_permutation(dtype, b_col):
    """A * I == A and A * P permutes the columns of A, exactly, on the GPU."""
    M, K = 200, 320
    lo, hi = (-128, 127) if dtype == "i8" else (-1, 1)
    A = I.draw("uniform", lo, hi, (M, K), np.random.default_rng(5), dtype)
    Av = parity.values(A, dtype)
    from tests.oracle_pins import _store
    eye = _store(np.eye(K), dtype)
    pi = [(k + 37) % K for k in range(K)]
    Pm = np.zeros((K, K))
    for k in range(K):
        Pm[k, pi[k]] = 1.0
    P = _store(Pm, dtype)
    for Bm, want in [(eye, Av), (P, Av[:, np.argsort(pi)])]:
        Bs = np.ascontiguousarray(Bm.T) if b_col else Bm
        C = run(A, Bs, dtype, b_col, M, K, K)
        assert np.array_equal(C.astype(np.float64), want)


def test_k_zero_writes_zeros():
    A = np.zeros((70, 8), dtype=np.uint16)
    B = np.zeros((1, 264), dtype=np.uint16)
    C = run(A, B, "f16", False, 70, 260, 0)
    assert np.all(C == 0)


def test_non_default_stream(oracle_mod):
    M, N, K = 256, 512, 512
    A, B = operands("bf16", False, M, N, K, 9)
    Cref = ref(oracle_mod, A, B, "bf16", False, N, K)
    dA, dB = to_dev(A, "bf16"), to_dev(B, "bf16")
    C = alloc_c(M, N, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        launch(dA, dB, C, "bf16", M, N, K, A.shape[1], B.shape[1], False, stream=s)
    s.synchronize()
    parity.check_full(C.cpu().numpy(), Cref, A, B, "bf16", False, M, N, K)


def test_torch_wrapper(oracle_mod):
    M, N, K = 130, 250, 96
    A, B = operands("f16", True, M, N, K, 13, pad_nan=False)
    Cref = ref(oracle_mod, A, B, "f16", True, N, K)
    out = spt.gemm(to_dev(A, "f16"), to_dev(B, "f16"), b_layout="col", K=K, N=N)
    torch.cuda.synchronize()
    parity.check_full(out.cpu().numpy(), Cref, A, B, "f16", True, M, N, K)


def test_torch_wrapper_rejects_unsafe_arguments():
    """The wrapper refuses, before any launch, what would make a kernel read or
    write outside the tensors: an output of the wrong dtype or device, K or N
    beyond the operands, operands on different devices."""
    A = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    B = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        spt.gemm(A, B, out=torch.zeros((64, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        spt.gemm(A, B, out=torch.zeros((64, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        spt.gemm(A, B, K=80)
    with pytest.raises(ValueError):
        spt.gemm(A, B, N=72)
    with pytest.raises(ValueError):
        spt.gemm(A, B, b_layout="col", N=65)
    with pytest.raises(ValueError):
        spt.gemm(A, B.cpu())
    with pytest.raises(ValueError):
        spt.gemm(A, B, b_layout="columns")
    C = spt.gemm(A, B, K=48, N=40)  # within the operands: fine
    assert tuple(C.shape) == (64, 40)


def test_launch_status_ignores_an_earlier_hip_error(oracle_mod):
    """A failed HIP call made before spt_gemm (here an allocation of 2^50 bytes,
    which the runtime refuses) leaves an error in the runtime's last-error slot;
    the library reports its own launch's status, and computes C."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMalloc.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    hip.hipPeekAtLastError.restype = ctypes.c_int
    A, B = operands("f16", False, 128, 256, 64, 9, pad_nan=False)
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    C = alloc_c(128, 256, "f16")
    torch.cuda.synchronize()
    p = ctypes.c_void_p()
    try:
        assert hip.hipMalloc(ctypes.byref(p), 1 << 50) != 0
        assert hip.hipPeekAtLastError() != 0
        rc = spt.spt_gemm(128, 256, 64, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1], C.data_ptr(),
                          C.stride(0), spt.F16, torch.cuda.current_stream().cuda_stream)
        assert rc == spt.SPT_OK, spt.spt_last_error()
    finally:
        hip.hipGetLastError()  # clear the slot for later tests
    torch.cuda.synchronize()
    parity.check_full(C.cpu().numpy(), ref(oracle_mod, A, B, "f16", False, 256, 64), A, B, "f16", False,
                      128, 256, 64)


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configurations the benchmark times;
# sampled outputs are recomputed one by one by the oracle.

def sampled(oracle_mod, w: I.Workload, variant="auto", stages=0, tile=0, n=3000):
    print(f"[gpu] full-size {w.name} {variant}/{stages} tile={tile}", flush=True)
    A, B = I.make_operands(w)
    dA, dB = to_dev(A, w.dtype), to_dev(B, w.dtype)
    C = alloc_c(w.M, w.N, w.dtype)
    launch(dA, dB, C, w.dtype, w.M, w.N, w.K, A.shape[1], B.shape[1], w.b_col, variant, stages, tile)
    rows, cols = parity.sample_entries(w.M, w.N, n, np.random.default_rng(w.wid))
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    # every output written: no sentinel anywhere
    if w.dtype == "i8":
        assert not bool((C == int(SENT_I)).any())
    else:
        assert bool(torch.isfinite(C).all())
    want = oracle_mod.gemm_entries(A, B, w.dtype, rows, cols, b_col=w.b_col, K=w.K)
    return parity.check_entries(got, want, rows, cols, A, B, w.dtype, w.b_col, w.M, w.N, w.K)


@pytest.mark.parametrize("variant,stages", [("auto", 0)] + PAIRS)
def test_full_fp16_4096(oracle_mod, variant, stages):
    sampled(oracle_mod, I.W_F16_4096, variant, stages, 1)


@pytest.mark.parametrize("tile,stages", [(2, 2), (2, 3), (4, 2), (4, 3), (5, 2), (5, 3), (5, 4), (1, 4), (6, 2)])
def test_full_fp16_4096_ring_tiles(oracle_mod, tile, stages):
    """The ring kernels of the other tiles at the full 4096^3 size (exact-fit,
    except the 256 x 192 tile, whose grid has a ragged last column)."""
    sampled(oracle_mod, I.W_F16_4096, "direct", stages, tile)


@pytest.mark.parametrize("variant,stages,tile", [("auto", 0, 0), ("sync", 1, 1), ("direct", 2, 1),
                                                 ("direct", 2, 4), ("direct", 3, 5)])
def test_full_int8_4096_bcol(oracle_mod, variant, stages, tile):
    sampled(oracle_mod, I.W_I8_4096, variant, stages, tile)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8", "f32"])
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("M,N,K", [(512, 768, 640), (256, 384, 128), (500, 700, 333)])
def test_tile_256x192_all_pairs(oracle_mod, dtype, b_col, M, N, K):
    """The 256 x 192 tile: shapes that are multiples of it (exact-fit kernels)
    and a ragged one (general kernels); every (variant, stages) pair agrees
    with the oracle and bit for bit with the others."""
    K = K if dtype != "f32" else K // 2
    A, B = operands(dtype, b_col, M, N, K, 13, lda_pad=0 if M % 256 == 0 else 8, ldb_pad=0 if M % 256 == 0 else 8)
    Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
    outs = []
    for v, st in PAIRS:
        if not built(6, v, st):
            continue
        C = run(A, B, dtype, b_col, M, N, K, v, st, 6)
        parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)
        outs.append(C)
    for C in outs[1:]:
        assert np.array_equal(C.view(np.uint32), outs[0].view(np.uint32)), (dtype, b_col, M, N, K)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 96), (512, 256, 128), (256, 512, 192)])
def test_exact_shapes_odd_and_even_k_tiles(oracle_mod, dtype, M, N, K):
    """Tile-multiple shapes whose count of 64-byte K tiles is odd (general
    kernel) or even (exact-fit kernel): every ring depth of the tiles with a
    64-byte K depth agrees with the oracle and bit for bit with SYNC."""
    A, B = operands(dtype, False, M, N, K, 11)
    Cref = ref(oracle_mod, A, B, dtype, False, N, K)
    for tile in (1, 3, 5):
        outs = []
        for v, s in [("sync", 1), ("direct", 2), ("direct", 3), ("direct", 4)]:
            C = run(A, B, dtype, False, M, N, K, v, s, tile)
            parity.check_full(C, Cref, A, B, dtype, False, M, N, K)
            outs.append(C)
        for C in outs[1:]:
            assert np.array_equal(C.view(np.uint32), outs[0].view(np.uint32)), (tile, M, N, K)


@pytest.mark.parametrize("K", I.LOWK_KS)
def test_full_bf16_lowk(oracle_mod, K):
    sampled(oracle_mod, I.w_bf16_lowk(K))


@pytest.mark.parametrize("w,tile", [
    (I.Workload("bf16 GEMM 3000x3000x3000", 31, "bf16", 3000, 3000, 3000), 6),
    (I.Workload("int8 GEMM 4000x3008x4000, B column-major", 32, "i8", 4000, 3008, 4000, True), 6),
    (I.Workload("fp16 GEMM 8000x2000x8000", 33, "f16", 8000, 2000, 8000), 2),
    (I.Workload("fp16 GEMM 4608x4608x4608", 34, "f16", 4608, 4608, 4608), 6),
    (I.Workload("int8 GEMM 4608x4608x4608, B column-major", 35, "i8", 4608, 4608, 4608, True), 6)],
    ids=["bf16_3000", "i8_4000x3008", "f16_8000x2000", "f16_4608", "i8_4608"])
def test_full_auto_large_tile_shapes(oracle_mod, w, tile):
    """Shapes on which the library's choice is an 8-wave tile: 256 x 192 where a
    256 x 256 grid would leave CUs idle in its one round or end in a partly filled
    round (4608^3, exact fit), 256 x 256 where it fills them (general kernels:
    edges and a K tail): sampled outputs against the oracle, int8 bit-exact."""
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[w.dtype], w.M, w.N, w.K, spt.COL if w.b_col else spt.ROW)
    assert rc == 0 and pi.tile_id == tile
    sampled(oracle_mod, w)


# ---- row band of a nearly empty last round (AUTO) ----------------------------
@pytest.mark.parametrize("dtype,b_col,K", [("f16", False, 1040), ("bf16", True, 1032), ("i8", True, 2100),
                                           ("i8", False, 2100), ("f32", False, 524)])
def test_row_band_full(oracle_mod, dtype, b_col, K):
    """4224 x 4000: 33 x 16 tiles of 128 x 256, one more row of tiles than two
    rounds of 512 hold; the last 128 rows run as a second grid of 128 x 128
    tiles.  Every output against the oracle (int8 bit-exact), nothing written
    past N, and bit-identical to the one-grid 128 x 256 kernel."""
    M, N = 4224, 4000
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW)
    assert rc == 0 and pi.band_tile == spt.TILE_128x128 and pi.band_m == 4096
    A, B = operands(dtype, b_col, M, N, K, 40)
    C = run(A, B, dtype, b_col, M, N, K)
    parity.check_full(C, ref(oracle_mod, A, B, dtype, b_col, N, K), A, B, dtype, b_col, M, N, K)
    C1 = run(A, B, dtype, b_col, M, N, K, "direct", 3, 1)
    assert np.array_equal(C.view(np.uint32), C1.view(np.uint32))


@pytest.mark.parametrize("dtype,b_col,K", [("i8", True, 8192), ("f32", False, 2048), ("bf16", True, 4096)])
def test_row_band_four_stages(oracle_mod, dtype, b_col, K):
    """A band of at most one workgroup per CU with at least 8 KiB of K per row runs a
    4-stage ring, for every element type (4224 x 4000: 32 workgroups of 128 x 128 in the
    band): every output against the oracle (int8 bit-exact), bit-identical to the
    one-grid 128 x 256 kernel."""
    M, N = 4224, 4000
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW)
    assert rc == 0 and pi.band_tile == spt.TILE_128x128 and pi.band_stages == 4 and pi.band_grid == 32
    A, B = operands(dtype, b_col, M, N, K, 44)
    C = run(A, B, dtype, b_col, M, N, K)
    parity.check_full(C, ref(oracle_mod, A, B, dtype, b_col, N, K), A, B, dtype, b_col, M, N, K)
    C1 = run(A, B, dtype, b_col, M, N, K, "direct", 3, 1)
    assert np.array_equal(C.view(np.uint32), C1.view(np.uint32))


@pytest.mark.parametrize("w", [I.Workload("fp16 GEMM 4100x4104x4104", 41, "f16", 4100, 4104, 4104),
                               I.Workload("int8 GEMM 4100x4112x4112, B column-major", 42, "i8", 4100, 4112, 4112,
                                          True),
                               I.Workload("fp16 GEMM 4352x4096x8192", 43, "f16", 4352, 4096, 8192)],
                         ids=["f16_4100", "i8_4100", "f16_4352"])
def test_full_row_band(oracle_mod, w):
    """Full-size shapes whose last rows the library runs as a band of 128 x 128
    tiles (after a 128 x 256 or a 256 x 256 grid): sampled outputs against the
    oracle."""
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[w.dtype], w.M, w.N, w.K, spt.COL if w.b_col else spt.ROW)
    assert rc == 0 and pi.band_tile == spt.TILE_128x128
    sampled(oracle_mod, w)


@pytest.mark.parametrize("variant,stages", [("auto", 0), ("reg", 2), ("sync", 1)])
def test_full_bf16_ragged(oracle_mod, variant, stages):
    sampled(oracle_mod, I.W_BF16_RAGGED, variant, stages)


# ---- maximum sizes ------------------------------------------------------------
@pytest.mark.parametrize("b_col", [False, True])
def test_int8_max_k_extremes_bit_exact(oracle_mod, b_col):
    """K = 131071, the largest K whose int32 sums are exact: rows of all -128
    against columns of all -128 reach 131071 * 16384 = 2147467264, just below
    2^31; mixed with random rows.  Bit-exact against the oracle."""
    M, N, K = 32, 48, 131071
    A, B = operands("i8", b_col, M, N, K, 21)
    A[:4, :K] = -128
    if b_col:
        B[:6, :K] = -128
    else:
        B[:K, :6] = -128
    Cref = ref(oracle_mod, A, B, "i8", b_col, N, K)
    assert Cref[0, 0] == 131071 * 16384
    for v, s in [("auto", 0), ("direct", 3), ("sync", 1)]:
        C = run(A, B, "i8", b_col, M, N, K, v, s)
        assert np.array_equal(C, Cref)


def test_fp16_very_long_k(oracle_mod):
    """K = 2^20: 32768 K tiles through the ring (plus a 7-wide tail)."""
    M, N, K = 16, 40, (1 << 20) + 7
    A, B = operands("f16", False, M, N, K, 22)
    C = run(A, B, "f16", False, M, N, K)
    parity.check_full(C, ref(oracle_mod, A, B, "f16", False, N, K), A, B, "f16", False, M, N, K)


def test_large_output_sampled(oracle_mod):
    """C of 16384 x 16384 fp32 (1 GiB) from K = 64: every output written, sampled
    entries against the oracle."""
    sampled(oracle_mod, I.Workload("fp16 GEMM 16384x16384x64", 23, "f16", 16384, 16384, 64), n=2000)


@pytest.mark.parametrize("dtype,b_col", [("bf16", False), ("i8", True), ("f32", False)])
@pytest.mark.parametrize("M,N,K", [(1, 70001, 300), (70001, 1, 300), (3, 5, 100003), (129, 40000, 40)])
def test_extreme_aspect_ratios(oracle_mod, dtype, b_col, M, N, K):
    """One row or one column of C across hundreds of tiles, a tiny C from a K of
    10^5 (thousands of K tiles and a ragged tail), and a wide C from a short K:
    full C against the oracle, under AUTO and the unpipelined loop."""
    A, B = operands(dtype, b_col, M, N, K, 300 + M % 97 + N % 89, lda_pad=1, ldb_pad=2)
    Cref = ref(oracle_mod, A, B, dtype, b_col, N, K)
    for v, s in (("auto", 0), ("sync", 1)):
        C = run(A, B, dtype, b_col, M, N, K, v, s)
        parity.check_full(C, Cref, A, B, dtype, b_col, M, N, K)


def _random_shapes(n=32):
    """Seeded shapes across element types and B layouts, large enough that AUTO picks
    every tile family (128 x 128 up to the 256 x 256 and 256 x 192 tiles)."""
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(n):
        dtype = ["f16", "bf16", "i8", "f32"][i % 4]
        b_col = bool((i // 4) % 2)
        M, N = (int(x) for x in rng.integers(1, 5200, 2))
        K = int(rng.integers(1, 3000 if dtype != "f32" else 800))
        out.append((dtype, b_col, M, N, K))
    return out


@pytest.mark.parametrize("dtype,b_col,M,N,K", _random_shapes())
def test_auto_random_shapes(oracle_mod, dtype, b_col, M, N, K):
    """AUTO on seeded random shapes, pitches padded to 16-byte multiples: sampled
    outputs against the oracle (int8 bit-exact), every output written and nothing
    written outside M x N."""
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW)
    assert rc == 0
    print(f"[gpu] random {dtype} {'col' if b_col else 'row'} {M}x{N}x{K} tile {pi.tile_id}", flush=True)
    A, B = operands(dtype, b_col, M, N, K, 40 + M % 50, pad_nan=False)
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    ldc = -(-(N + 1) // 4) * 4  # a 16-byte pitch with at least one padding column
    C = alloc_c(M, ldc, dtype)
    launch(dA, dB, C, dtype, M, N, K, A.shape[1], B.shape[1], b_col)
    sent = int(SENT_I) if dtype == "i8" else int(np.array(SENT_F).view(np.int32))
    raw = C.view(torch.int32)
    assert bool((raw[:, N:] == sent).all()), "write outside M x N"
    assert not bool((raw[:, :N] == sent).any()), "output left unwritten"
    rows, cols = parity.sample_entries(M, N, 600, np.random.default_rng(M * 7 + N))
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    want = oracle_mod.gemm_entries(A, B, dtype, rows, cols, b_col=b_col, K=K)
    parity.check_entries(got, want, rows, cols, A, B, dtype, b_col, M, N, K)
