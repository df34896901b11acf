"""The C-ABI library without a GPU: it loads, exports every declared entry point,
rejects bad arguments before touching a device, and its planner agrees with the
pages' formulas (restated in oracle/plan_oracle.py)."""
import ctypes
import os
import re

import pytest

import software_pipelined_tiling_amd as spt
from oracle import plan_oracle as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L(built_lib):
    return spt.lib()


def declared_functions():
    inc = os.path.join(ROOT, "include")
    txt = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(spt_\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert names == sorted(["spt_gemm", "spt_gemm_ex", "spt_plan", "spt_status_string",
                            "spt_last_error", "spt_version", "spt_scale_by_two", "spt_attention"])
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert spt.spt_version() == 10100
    assert spt.spt_status_string(0) == "SPT_OK"
    assert spt.spt_status_string(-1) == "SPT_ERR_INVALID"
    assert spt.spt_status_string(-2) == "SPT_ERR_UNSUPPORTED"
    assert spt.spt_status_string(-3) == "SPT_ERR_MISALIGNED"
    assert spt.spt_status_string(-4) == "SPT_ERR_LAUNCH"
    assert spt.spt_status_string(99) == "SPT_ERR_UNKNOWN"


# Fake but aligned device addresses: every call below must fail validation
# before any HIP call, so nothing is ever dereferenced.
PA, PB, PC = 0x10000, 0x20000, 0x30000


def ex(M=64, N=64, K=64, A=PA, lda=None, B=PB, ldb=None, C=PC, ldc=None, dtype=spt.F16, lay=spt.ROW,
       var=spt.VARIANT_AUTO, st=0, tile=0):
    lda = K if lda is None else lda
    ldb = (K if lay == spt.COL else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return spt.spt_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, 0, lay, var, st, tile)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), -1), (dict(lay=2), -1), (dict(var=9), -1), (dict(st=5), -1), (dict(tile=9), -1),
    (dict(M=-1), -1), (dict(K=-5), -1), (dict(C=0), -1), (dict(A=0), -1), (dict(B=0), -1),
    (dict(lda=32), -1), (dict(ldb=32), -1), (dict(ldc=8), -1), (dict(lay=spt.COL, ldb=32), -1),
    (dict(var=spt.VARIANT_SYNC, st=2), -2), (dict(var=spt.VARIANT_DIRECT, st=1), -2),
    (dict(var=spt.VARIANT_REG, st=3), -2), (dict(dtype=spt.I8, K=131072), -2),
    (dict(var=spt.VARIANT_DIRECT, st=4, tile=spt.TILE_256x256_4W), -2), (dict(tile=7), -1),
    (dict(var=spt.VARIANT_DIRECT, st=3, tile=spt.TILE_256x192), -2),
    (dict(var=spt.VARIANT_DIRECT, st=4, tile=spt.TILE_256x256), -2),
    (dict(A=0x8000), -2), (dict(B=1 << 47), -2),
    (dict(A=PA + 8), -3), (dict(B=PB + 2), -3), (dict(C=PC + 4), -3),
    (dict(K=60, lda=60), -3), (dict(N=60, ldb=60, ldc=64), -3), (dict(N=62, ldc=62), -3),
])
def test_validation_errors(L, kw, status):
    assert ex(**kw) == status
    assert spt.spt_last_error() != ""


@pytest.mark.parametrize("kw", [dict(C=PA), dict(C=PA + 0x1000), dict(C=PB), dict(C=PB + 0x1FF0),
                                dict(C=PA - 0x3FF0), dict(lay=spt.COL, C=PB + 0x10)])
def test_output_overlapping_an_operand_is_refused(L, kw):
    """C written while A and B are read: any shared byte is refused before a launch
    (a C starting 16 bytes less than its size below A ends inside A's first row)."""
    assert ex(**kw) == -1
    assert "overlap" in spt.spt_last_error()


def test_too_many_output_tiles_is_refused(L):
    assert ex(M=1 << 30, N=(1 << 31) - 16, ldc=(1 << 31) - 16) == -2


def test_empty_problem_is_ok_without_launch(L):
    assert ex(M=0) == 0
    assert ex(N=0, ldb=1, ldc=1) == 0
    assert spt.spt_gemm(0, 0, 0, 0, 1, 0, 1, 0, 1, spt.F16, 0) == 0


def test_plan_rejects_what_gemm_rejects(L):
    rc, _ = spt.spt_plan(spt.I8, 64, 64, 200000)
    assert rc == -2
    rc, _ = spt.spt_plan(5, 64, 64, 64)
    assert rc == -1
    assert L.spt_plan(0, 1, 1, 1, 0, 0, 0, 0, None) == -1


DTYPES = [(spt.F16, 2), (spt.BF16, 2), (spt.I8, 1), (spt.F32, 4)]
PAIRS = [(spt.VARIANT_SYNC, 1), (spt.VARIANT_REG, 1), (spt.VARIANT_REG, 2), (spt.VARIANT_DIRECT, 2),
         (spt.VARIANT_DIRECT, 3), (spt.VARIANT_DIRECT, 4)]
TILES = {1: (128, 256, 64, 256), 2: (256, 256, 128, 512), 3: (128, 128, 64, 256), 4: (256, 256, 128, 256),
         5: (256, 256, 64, 256), 6: (256, 192, 128, 512)}


@pytest.mark.parametrize("dtype,elt", DTYPES)
@pytest.mark.parametrize("tile", sorted(TILES))
@pytest.mark.parametrize("var,st", PAIRS)
def test_plan_matches_page_formulas(L, dtype, elt, tile, var, st):
    BM, BN, BKB, thr = TILES[tile]
    BK = BKB // elt
    M, N, K = 4000, 3000, 1000
    rc, pi = spt.spt_plan(dtype, M, N, K, spt.ROW, var, st, tile)
    half = BM * BKB  # bytes of one operand's part of a stage
    if P.ring_bytes(BM, BN, BKB // elt, elt, st) > 163840:  # the ring does not fit in LDS
        if var == spt.VARIANT_DIRECT and BM == BN and (2 * st - 1) * half <= 163840:
            # ... but its 2S - 1 half stages do (A and B parts of one size)
            assert rc == 0 and pi.half_stage_slots == 2 * st - 1 and pi.lds_bytes == (2 * st - 1) * half
            assert pi.steady_vmcnt == (2 * st - 5) * pi.a_copies_per_thread
            assert pi.a_copies_per_thread == pi.b_copies_per_thread == P.copies_per_thread(BM, BKB // elt, elt, thr)
            return
        assert rc == -2
        return
    assert pi.half_stage_slots == 0
    assert rc == 0
    assert (pi.BM, pi.BN, pi.BK, pi.threads) == (BM, BN, BK, thr)
    assert pi.stage_bytes == P.stage_bytes(BM, BN, BK, elt)
    assert pi.a_stage_bytes == BM * BK * elt and pi.b_stage_bytes == BK * BN * elt
    assert pi.lds_bytes == P.ring_bytes(BM, BN, BK, elt, st)
    assert pi.a_copies_per_thread == P.copies_per_thread(BM, BK, elt, thr)
    assert pi.b_copies_per_thread == P.copies_per_thread(BK, BN, elt, thr)
    assert pi.ratio_flop_per_byte == pytest.approx(P.compute_load_ratio(BM, BN, BK, elt), rel=1e-12)
    gfx950 = P.Machine(regs_per_sm=4 * 512 * 64, smem_per_sm=163840, max_warps_per_sm=32,
                       max_blocks_per_sm=32, warp_size=64)
    blocks, _, lim = P.occupancy(gfx950, 0, pi.lds_bytes, thr)
    assert pi.wg_per_cu_lds == lim["smem"]
    assert pi.tiles_m == -(-M // BM) and pi.tiles_n == -(-N // BN) and pi.grid == pi.tiles_m * pi.tiles_n
    assert pi.k_tiles == -(-K // BK) and pi.k_full_tiles == K // BK and pi.k_tail == K % BK
    expect_vm = (st - 2) * (pi.a_copies_per_thread + pi.b_copies_per_thread) if var == spt.VARIANT_DIRECT else 0
    assert pi.steady_vmcnt == expect_vm


def test_pages_tile_plan(L):
    """The 128 x 256 x 32 fp16 tile with 256 threads and 3 stages: 24 KiB per stage,
    72 KiB in all, 2 + 4 sixteen-byte copies per thread per stage."""
    rc, pi = spt.spt_plan(spt.F16, 4096, 4096, 4096, spt.ROW, spt.VARIANT_DIRECT, 3, 1)
    assert rc == 0
    assert (pi.stage_bytes, pi.lds_bytes) == (24576, 73728)
    assert (pi.a_copies_per_thread, pi.b_copies_per_thread) == (2, 4)
    assert pi.wg_per_cu_lds == 2 and pi.steady_vmcnt == 6
    assert pi.grid == 512 and pi.k_tiles == 128


# ---- the library's choice (AUTO) ------------------------------------------------
@pytest.mark.parametrize("dtype,M,N,K,lay,tile,stages", [
    (spt.F16, 4096, 4096, 4096, spt.ROW, 4, 2),     # exact 256 x 256, long K
    (spt.F16, 8192, 8192, 8192, spt.ROW, 4, 2),
    (spt.F16, 5120, 5120, 4096, spt.ROW, 4, 2),
    (spt.F16, 7168, 7168, 4096, spt.ROW, 4, 2),
    (spt.F16, 4608, 4608, 4608, spt.ROW, 6, 2),     # a partly filled last round of 256 x 256
    (spt.F16, 6144, 6144, 6144, spt.ROW, 6, 2),
    (spt.BF16, 6144, 6144, 2048, spt.ROW, 6, 2),
    (spt.F16, 4096, 6144, 4096, spt.ROW, 6, 2),
    (spt.I8, 4608, 4608, 4608, spt.COL, 6, 2),
    (spt.I8, 5120, 5120, 4096, spt.COL, 4, 2),
    (spt.I8, 4608, 4608, 4608, spt.ROW, 6, 2),
    (spt.I8, 4096, 4096, 4096, spt.COL, 4, 2),
    (spt.BF16, 8192, 8192, 512, spt.ROW, 1, 3),     # low K: the C store decides
    (spt.BF16, 8192, 8192, 128, spt.ROW, 1, 3),     # four K tiles: the ring
    (spt.F16, 256, 256, 256, spt.ROW, 3, 3),        # too few 128 x 256 tiles for the CUs
    (spt.BF16, 4000, 3000, 1000, spt.ROW, 6, 2),    # 256 x 256 would leave CUs idle in its one
    (spt.BF16, 3000, 3000, 3000, spt.ROW, 6, 2),    # round; 256 x 192 still fits one round
    (spt.I8, 4000, 3008, 4000, spt.COL, 6, 2),
    (spt.BF16, 2048, 6144, 2048, spt.ROW, 6, 2),
    (spt.BF16, 4096, 3072, 1024, spt.ROW, 6, 2),
    (spt.F16, 5000, 5000, 1024, spt.ROW, 2, 2),     # 256 x 256 tiles over more than one round
    (spt.F16, 8000, 2000, 8000, spt.ROW, 2, 2),     # ... or exactly one round of all CUs
    (spt.BF16, 2000, 4000, 1000, spt.ROW, 1, 3),    # 256 x 256 would leave half the CUs idle
    (spt.F16, 4100, 4100, 4100, spt.ROW, 1, 3),     # ... or a long partial round
    (spt.F16, 6000, 6000, 2000, spt.ROW, 1, 3),
])
def test_auto_choice(L, dtype, M, N, K, lay, tile, stages):
    """AUTO's tile and ring depth on shapes measured on MI355X (the comment above
    resolve() in csrc/spt_api.cpp gives the measurements)."""
    rc, pi = spt.spt_plan(dtype, M, N, K, lay)
    assert rc == 0, spt.spt_last_error()
    assert (pi.tile_id, pi.variant, pi.stages) == (tile, spt.VARIANT_DIRECT, stages)


@pytest.mark.parametrize("dtype,M,N,K,lay,variant", [
    (spt.BF16, 8192, 8192, 32, spt.ROW, spt.VARIANT_SYNC),   # one or two K tiles, four rounds or more
    (spt.BF16, 8192, 8192, 64, spt.ROW, spt.VARIANT_SYNC),
    (spt.F16, 8192, 8192, 64, spt.ROW, spt.VARIANT_SYNC),
    (spt.I8, 8192, 8192, 128, spt.COL, spt.VARIANT_SYNC),
    (spt.BF16, 8192, 8192, 40, spt.ROW, spt.VARIANT_SYNC),   # one partial K tile
    (spt.BF16, 4096, 4096, 64, spt.ROW, spt.VARIANT_DIRECT),  # one round
    (spt.BF16, 6144, 6144, 64, spt.ROW, spt.VARIANT_DIRECT),  # 2.25 rounds
    (spt.F16, 8192, 4096, 64, spt.ROW, spt.VARIANT_DIRECT),   # two rounds
    (spt.F32, 8192, 8192, 32, spt.ROW, spt.VARIANT_DIRECT),   # fp32 keeps the ring
    (spt.BF16, 8192, 8192, 96, spt.ROW, spt.VARIANT_DIRECT),  # three K tiles
    (spt.BF16, 8192, 8192, 0, spt.ROW, spt.VARIANT_DIRECT),   # nothing to load
])
def test_auto_variant_at_short_k(L, dtype, M, N, K, lay, variant):
    """With one or two K tiles AUTO takes the unpipelined loop where it was measured
    faster (a store-bound grid of four or more rounds); the ring elsewhere."""
    rc, pi = spt.spt_plan(dtype, M, N, K, lay)
    assert rc == 0, spt.spt_last_error()
    assert pi.variant == variant
    assert pi.stages == (1 if variant == spt.VARIANT_SYNC else 3)
    # an explicit stage count or variant is never overridden
    rc, pi = spt.spt_plan(dtype, M, N, K, lay, spt.VARIANT_AUTO, 3, 0)
    assert rc == 0 and pi.variant == spt.VARIANT_DIRECT


# ---- the persistent variant ---------------------------------------------------
@pytest.mark.parametrize("K,window", [(64, 2), (128, 4), (192, 4), (256, 8), (512, 8), (4096, 8)])
def test_persist_plan(L, K, window):
    """bf16 8192 x 8192: 4096 tiles of 128 x 128 over 512 persistent workgroups
    (two per CU), eight each; the store window is the longest of 2, 4, 8 K tiles
    that fits; the steady wait leaves the younger copies and the stores
    issued after the awaited copies in flight."""
    rc, pi = spt.spt_plan(spt.BF16, 8192, 8192, K, spt.ROW, spt.VARIANT_PERSIST, 0, 0)
    assert rc == 0, spt.spt_last_error()
    assert (pi.tile_id, pi.stages, pi.BM, pi.BN, pi.BK) == (3, 3, 128, 128, 32)
    assert pi.grid == 512 and pi.tiles_per_wg == 8 and pi.store_window == window
    assert pi.lds_bytes == 3 * 16384
    assert pi.steady_vmcnt == 1 * 4 + 2 * (16 // window)


def test_persist_plan_small_grid_and_errors(L):
    rc, pi = spt.spt_plan(spt.F16, 384, 512, 64, spt.ROW, spt.VARIANT_PERSIST, 2, 3)
    assert rc == 0 and pi.grid == 12 and pi.tiles_per_wg == 1
    rc, pi = spt.spt_plan(spt.F16, 4096, 4096, 64, spt.ROW, spt.VARIANT_DIRECT, 3, 1)
    assert rc == 0 and pi.store_window == 0 and pi.tiles_per_wg == 1
    assert spt.spt_plan(spt.F16, 512, 512, 64, spt.ROW, spt.VARIANT_PERSIST, 3, 1)[0] == -2
    assert spt.spt_plan(spt.F16, 512, 512, 64, spt.ROW, spt.VARIANT_PERSIST, 1, 0)[0] == -2


@pytest.mark.parametrize("M,N,K,st,tile", [
    (100, 256, 64, 3, 0), (128, 200, 64, 3, 0), (128, 256, 70, 3, 0), (128, 256, 96, 3, 0),
    (128, 256, 32, 3, 0), (128, 256, 64, 4, 0), (128, 256, 64, 3, 1), (128, 256, 0, 3, 0)])
def test_persist_rejects_unfit_shapes(L, M, N, K, st, tile):
    """Outside its scope (a ragged M or N, a K tail, an odd count of K tiles, one
    K tile, a 4-stage ring over 2 K tiles, another tile, K = 0) the persistent
    variant returns SPT_ERR_UNSUPPORTED before any HIP call."""
    assert ex(M=M, N=N, K=K, lda=max(8, -(-K // 8) * 8), var=spt.VARIANT_PERSIST, st=st, tile=tile) == -2
    assert spt.spt_last_error() != ""


# ---- the streaming pipeline y = 2x: validation before any HIP call -----------
X0, Y0 = 0x100000, 0x200000   # fake, aligned, far apart


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), -1), (dict(stages=5), -1), (dict(stages=-1), -1), (dict(blocks=-2), -1),
    (dict(x=0), -1), (dict(y=0), -1), (dict(y=X0 + 4), -1),          # partial overlap
    (dict(x=X0 + 4, y=X0 + 4 + (1 << 20)), -3), (dict(y=Y0 + 8), -3),  # misaligned
    (dict(x=0x8000, y=0x9000 + (1 << 20)), -2), (dict(y=1 << 47), -2), (dict(n=(1 << 40) + 1), -2),
])
def test_scale_by_two_validation(L, kw, status):
    a = dict(n=1000, x=X0, y=Y0, stages=0, blocks=0)
    a.update(kw)
    assert spt.spt_scale_by_two(a["n"], a["x"], a["y"], a["stages"], a["blocks"], 0) == status
    assert spt.spt_last_error() != ""


def test_scale_by_two_empty_is_ok(L):
    assert spt.spt_scale_by_two(0, 0, 0, 0, 0, 0) == 0


def test_panel_above_2gib_is_refused(L):
    """A 256-row panel of A with a 2^22-element fp16 pitch is 2 GiB of buffer
    offsets: refused before any launch."""
    K = 1 << 22
    assert ex(M=256, N=256, K=K, lda=K, tile=spt.TILE_256x256_4W) == -2
    assert "2 GiB" in spt.spt_last_error()


QA, KA, VA, OA = 0x1000000, 0x2000000, 0x3000000, 0x4000000  # fake, aligned, far apart


@pytest.mark.parametrize("kw,status", [
    (dict(BH=-1), spt.SPT_ERR_INVALID), (dict(Sk=0), spt.SPT_ERR_INVALID), (dict(scale=-1.0), spt.SPT_ERR_INVALID),
    (dict(variant=4), spt.SPT_ERR_INVALID), (dict(stages=5), spt.SPT_ERR_INVALID),
    (dict(D=96), spt.SPT_ERR_UNSUPPORTED), (dict(dtype=spt.I8), spt.SPT_ERR_UNSUPPORTED),
    (dict(variant=spt.VARIANT_SYNC, stages=2), spt.SPT_ERR_UNSUPPORTED),
    (dict(variant=spt.VARIANT_DIRECT, stages=1), spt.SPT_ERR_UNSUPPORTED),
    (dict(Q=0), spt.SPT_ERR_INVALID), (dict(O=KA + 64), spt.SPT_ERR_INVALID),   # null, O overlaps K
    (dict(K=KA + 8), spt.SPT_ERR_MISALIGNED),
    # one slice's K of 2^31 + 256 bytes (the kernel's 32-bit buffer offsets): refused
    (dict(BH=1, Sk=(1 << 23) + 1, D=128), spt.SPT_ERR_UNSUPPORTED),
    (dict(BH=1, Sk=(1 << 24) + 1, D=64), spt.SPT_ERR_UNSUPPORTED),
])
def test_attention_validation(L, kw, status):
    """spt_attention refuses bad arguments before any device call (fake pointers)."""
    a = dict(BH=2, Sq=64, Sk=64, D=64, Q=QA, K=KA, V=VA, O=OA, scale=0.125, dtype=spt.F16, variant=0, stages=0)
    a.update(kw)
    assert spt.spt_attention(a["BH"], a["Sq"], a["Sk"], a["D"], a["Q"], a["K"], a["V"], a["O"], a["scale"],
                             a["dtype"], 0, a["variant"], a["stages"]) == status
    assert spt.spt_last_error() != ""
    if kw.get("Sk", 0) > (1 << 22):
        assert "2^31 bytes" in spt.spt_last_error()


def test_last_error_describes_the_most_recent_call():
    """spt_last_error() holds a message after a refused call and is empty after any
    call that returned SPT_OK, including calls with nothing to launch."""
    assert spt.spt_plan(9, 64, 64, 64)[0] == spt.SPT_ERR_INVALID
    assert "dtype 9" in spt.spt_last_error()
    assert spt.spt_plan(spt.F16, 64, 64, 64)[0] == spt.SPT_OK
    assert spt.spt_last_error() == ""
    assert spt.spt_gemm(-1, 1, 1, 0, 1, 0, 1, 0, 1, spt.F16, 0) == spt.SPT_ERR_INVALID
    assert spt.spt_last_error() != ""
    assert spt.spt_gemm(0, 64, 64, 0, 64, 0, 64, 0, 64, spt.F16, 0) == spt.SPT_OK  # M = 0: no launch
    assert spt.spt_last_error() == ""
    assert spt.spt_scale_by_two(-1, 0, 0) == spt.SPT_ERR_INVALID
    assert spt.spt_scale_by_two(0, 0, 0) == spt.SPT_OK
    assert spt.spt_last_error() == ""


@pytest.mark.parametrize("dtype,M,N,K,b_col,band_m", [
    ("f16", 4100, 4104, 4104, False, 3840),
    ("i8", 4100, 4112, 4112, True, 3840),
    ("bf16", 6000, 6000, 2000, False, 5376),
    ("f32", 4100, 4100, 1024, False, 3840),
    ("bf16", 8448, 8192, 2048, False, 8192),  # 256 x 256 main grid
    ("f16", 4352, 4096, 8192, False, 4096),
    ("f16", 4224, 4000, 520, False, None),    # K below 2 KiB per row
    ("f16", 4096, 4096, 4096, False, None),   # full rounds
    ("f16", 5120, 5120, 4096, False, None),   # last round more than half full
    ("bf16", 4000, 3000, 1000, False, None),  # one round
    ("f16", 512, 102408, 4096, False, None),  # rows of 401 tiles leave the main grid a partial round
    ("f16", 4864, 5120, 4096, False, None),   # a band of 560 workgroups of 128 x 128
])
def test_row_band_plan(dtype, M, N, K, b_col, band_m):
    """A last round at most half full: the rows of tiles that fit the earlier
    rounds run as one grid, the rows below them as a second grid of 128 x 128
    tiles."""
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW)
    assert rc == 0
    if band_m is None:
        assert (pi.band_tile, pi.band_stages, pi.band_m, pi.band_grid) == (0, 0, M, 0)
        assert pi.grid == pi.tiles_m * pi.tiles_n
        return
    cap = 256 * min(2, 163840 // pi.lds_bytes)
    assert (pi.band_tile, pi.band_m) == (spt.TILE_128x128, band_m)
    total = pi.tiles_m * pi.tiles_n
    rounds = -(-total // cap)
    assert 2 * (total - (rounds - 1) * cap) <= cap           # last round at most half full
    assert band_m % pi.BM == 0 and pi.grid == band_m // pi.BM * pi.tiles_n
    assert (rounds - 1) * cap - pi.tiles_n < pi.grid <= (rounds - 1) * cap  # as many whole rows as fit
    assert (rounds - 1) * cap - pi.grid <= cap // 8 and pi.band_grid <= 512
    assert pi.band_stages == (4 if pi.band_grid <= 256 and K * pi.elt_bytes >= 8192 else 3)
    assert pi.band_grid == -(-(M - band_m) // 128) * -(-N // 128)
    # explicit requests never split
    rc, pe = spt.spt_plan(spt.DTYPE_CODES[dtype], M, N, K, spt.COL if b_col else spt.ROW, spt.VARIANT_DIRECT, 3, 1)
    assert rc == 0 and pe.band_tile == 0 and pe.grid == pe.tiles_m * pe.tiles_n


def test_plan_info_mirror_matches_the_c_layout(tmp_path):
    """The ctypes mirror of spt_plan_info has the C struct's size and every
    field at the C offset (gcc on include/spt.h)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    fields = [f for f, _ in spt.PlanInfo._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "spt.h"\nint main(void) {\n'
                   '    printf("size %zu\\n", sizeof(spt_plan_info));\n'
                   + "".join(f'    printf("{f} %zu\\n", offsetof(spt_plan_info, {f}));\n' for f in fields)
                   + "    return 0;\n}\n")
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(root, "include"), "-o", str(exe), str(src)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                      check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(spt.PlanInfo)
    for f in fields:
        assert int(got[f]) == getattr(spt.PlanInfo, f).offset, f


@pytest.mark.parametrize("dtype,M,N,K,lay,variant,stages,tile,want", [
    (spt.BF16, 4000, 3000, 1000, spt.ROW, 0, 0, 0, 1),   # the ragged workload: a 40-wide tail, 80 bytes
    (spt.BF16, 4000, 3000, 333, spt.ROW, 0, 0, 0, 0),    # 13 elements: not whole chunks
    (spt.I8, 300, 600, 64 * 5 + 16, spt.COL, 3, 2, 1, 1),
    (spt.I8, 300, 600, 64 * 5 + 8, spt.COL, 3, 2, 1, 0),
    (spt.F32, 300, 600, 16 * 4 + 4, spt.ROW, 3, 3, 3, 1),
    (spt.F16, 300, 600, 40, spt.ROW, 3, 3, 1, 1),        # no full tile: only the partial one
    (spt.F16, 300, 600, 40, spt.ROW, 1, 1, 1, 0),        # SYNC and REG keep the VGPR tail
    (spt.F16, 300, 600, 40, spt.ROW, 2, 2, 1, 0),
    (spt.F16, 600, 600, 72, spt.ROW, 3, 2, 2, 0),        # the 256 x 256 tiles keep it too
    (spt.F16, 600, 600, 72, spt.ROW, 3, 2, 4, 0),
    (spt.F16, 600, 600, 72, spt.ROW, 3, 2, 6, 1),
    (spt.F16, 512, 512, 512, spt.ROW, 3, 2, 1, 0),       # no partial tile
])
def test_tail_ring_plan(L, dtype, M, N, K, lay, variant, stages, tile, want):
    rc, pi = spt.spt_plan(dtype, M, N, K, lay, variant, stages, tile)
    assert rc == 0, spt.spt_last_error()
    assert pi.tail_ring == want
    if want:
        assert (pi.k_tail * pi.elt_bytes) % 16 == 0 and pi.k_tail > 0
