"""Disassembly checks of the shipped gfx950 kernels (no GPU needed).

The machine code in libspt.so must show the schedule the ring promises:
copies of later tiles issued between the MFMAs of the current one, the
steady-state vmcnt wait leaving (S-2) tiles of copies in flight, partial
lgkmcnt waits for the LDS -> VGPR fragment pipeline, one barrier per K tile,
no spills or accumulator copies inside the loop, and the LDS ring size of the
plan ("Pipeline GPU Kernel", Schritt 4: check in the generated code that the
next tile's loads are in flight during the math of the current one).
"""
import os
import re
import shutil

import pytest

from software_pipelined_tiling_amd import isa_check as X

pytestmark = pytest.mark.skipif(not os.path.exists(os.path.join(X.LLVM, "llvm-objdump")),
                                reason="ROCm llvm-objdump not installed")


@pytest.fixture(scope="module")
def kernels(built_lib):
    ks = X.load()
    assert ks, "no gemm kernels found in libspt.so"
    return ks


def pick(ks, **kw):
    out = [k for k in ks if all(getattr(k, a) == v for a, v in kw.items())]
    assert out, kw
    return out


def test_every_built_entry_is_in_the_binary(kernels):
    # 8 tables (element type x B layout) of 58: SYNC, REG 1/2 and DIRECT 2 on every tile,
    # DIRECT 3/4 where the ring fits in LDS (tiles 1, 3, 5), exact-fit forms of all of
    # these on tiles 1, 2, 4, 5 and 6, and DIRECT 3 as half-stage slots on tiles 2 and 4
    # (general and exact-fit)
    assert len(kernels) == 8 * 58
    assert {k.tile for k in kernels} == {1, 2, 3, 4, 5, 6}


@pytest.mark.parametrize("dtype", [0, 1])
def test_fp16_bf16_exact_rings_pass_every_check(kernels, dtype):
    for k in pick(kernels, dtype=dtype, variant="direct", exact=True):
        res = X.check(k)
        if k.geometry["half_stage_slots"]:
            # the half-stage ring's loop carries some accumulators across its back edge in
            # other registers (AGPR copies; its own test checks the schedule)
            res.pop("clean")
        assert all(res.values()), (k.name, res, X.loop_stats(k))


def test_headline_kernel_schedule(kernels):
    """256 x 256, 2-stage ring, fp16, row-major B, exact fit: 128 MFMAs and 16
    copies per K tile, one barrier, the copies one per MFMA gap, the wait before
    the barrier drains only the tile about to be read (vmcnt(0) with 2 stages)."""
    (k,) = pick(kernels, dtype=0, bcol=False, tile=4, variant="direct", stages=2, exact=True)
    st = X.loop_stats(k)
    assert (st["mfma"], st["dma"], st["barriers"]) == (128, 16, 1)
    assert st["vmcnt_waits"] == [0]
    assert st["dma_per_gap_max"] == 1 and st["dma_in_barrier_gap"] == 0
    assert st["scratch"] == 0 and st["acc_moves"] == 0
    assert k.meta["lds"] == 131072 and k.meta["agpr"] == 256 and k.meta["vgpr_spill"] == 0


@pytest.mark.parametrize("dtype,bcol", [(0, False), (1, False), (2, True), (2, False)])
@pytest.mark.parametrize("tile,half", [(4, 8), (2, 4)])
def test_half_stage_ring_schedule(kernels, dtype, bcol, tile, half):
    """The 3-stage ring of the 256 x 256 x 128-byte tiles in 5 half-stage slots (160 KiB):
    per K tile all copies and one barrier, and one wait that leaves one half stage of
    copies in flight (vmcnt(copies per tile / 2)), never vmcnt(0) in the steady loop;
    no scratch."""
    (k,) = pick(kernels, dtype=dtype, bcol=bcol, tile=tile, variant="direct", stages=3, exact=True)
    st = X.loop_stats(k)
    assert (st["dma"], st["barriers"]) == (2 * half, 1)
    assert st["vmcnt_waits"] == [half]
    assert st["dma_per_gap_max"] == 1 and st["dma_in_barrier_gap"] == 0 and st["scratch"] == 0
    assert k.meta["lds"] == 163840 and k.meta["vgpr_spill"] == 0
    assert k.geometry["half_stage_slots"] == 5 and X.check(k)["vmcnt"] and X.check(k)["lds"]


@pytest.mark.parametrize("tile,stages,loads", [(5, 3, 8), (5, 4, 8), (1, 3, 6), (1, 4, 6), (3, 3, 4)])
def test_deep_rings_keep_copies_in_flight(kernels, tile, stages, loads):
    """With S >= 3 the steady loop never waits for all copies: every vmcnt wait
    leaves the (S-2) younger tiles' copies in flight."""
    # (the general 256 x 256 kernels carry edge and tail code and spill in their loop;
    # scratch loads count in vmcnt too, so only their exact-fit forms are checked here)
    for k in pick(kernels, dtype=0, tile=tile, variant="direct", stages=stages):
        if tile in (4, 5) and not k.exact:
            continue
        st = X.loop_stats(k)
        assert st["vmcnt_waits"] and all(v == (stages - 2) * loads for v in st["vmcnt_waits"]), st
        assert 0 not in st["vmcnt_waits"]


def test_every_ring_has_the_planned_structure(kernels):
    """Counts (MFMAs, copies, barriers per loop iteration) and the LDS ring size
    hold for every DIRECT kernel of every element type and layout."""
    for k in pick(kernels, variant="direct"):
        res = X.check(k)
        assert res["counts"] and res["lds"], (k.name, res, X.loop_stats(k))


def test_small_tile_rings_are_clean(kernels):
    """Tiles with two waves per SIMD (1, 2, 3) keep accumulators in VGPRs: no
    spills or register copies in any of their ring loops, general or exact."""
    for k in kernels:
        if k.variant == "direct" and k.tile in (1, 2, 3) and k.stages <= 3:
            st = X.loop_stats(k)
            assert st["scratch"] == 0 and st["acc_moves"] == 0, (k.name, st)


def test_sync_loop_does_not_overlap(kernels):
    """The unpipelined reference drains its loads before its first MFMA."""
    for k in pick(kernels, variant="sync"):
        res = X.check(k)
        assert res["no_overlap"] and res["lds"], (k.name, res)


def test_register_staged_prefetch_overlaps(kernels):
    """REG issues tile t+1's global loads before tile t's first MFMA and waits
    for them only after its last one."""
    for k in pick(kernels, variant="reg"):
        res = X.check(k)
        assert all(res.values()), (k.name, res, X.loop_stats(k))


def test_cyclic_gaps_on_a_toy_loop():
    body = ["s_barrier", "v_mfma a", "buffer_load x lds", "v_mfma b", "ds_read_b128 y", "ds_read_b128 z"]
    assert X.cyclic_gaps(body) == [["buffer_load x lds"], ["ds_read_b128 y", "ds_read_b128 z", "s_barrier"]]


def test_streaming_ring_schedule(built_lib):
    """y = 2x ("Hiding Memory Latency ...", section 8): one copy, one store and one
    barrier per tile, and the steady wait vmcnt(2S-3) that leaves the S-1 younger
    copies and their stores in flight (S = 1: vmcnt(0) and two barriers)."""
    ks = X.load_stream()
    assert sorted(k.stages for k in ks) == [1, 2, 3, 4]
    for k in ks:
        res = X.check_stream(k)
        assert all(res.values()), (k.name, res)


def test_attention_schedule(built_lib):
    """The attention consumer (both element types, head dimension 64 and 128, every
    producer): per key block the MFMAs of both products; DIRECT's copies, one barrier
    and one vmcnt((S-2) x copies) wait; REG's loads overlapped with MFMAs before their
    vmcnt(0); SYNC's vmcnt(0) before any MFMA; no scratch; no accumulator-register
    copies in the loop; the LDS ring of S stages."""
    ks = X.load_attention()
    assert sorted({(k.dtype, k.D, k.variant, k.stages) for k in ks}) == sorted(
        (dt, d, v, s) for dt in (0, 1) for d in (64, 128)
        for v, s in (("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2), ("direct", 3)))
    for k in ks:
        res = X.check_attention(k)
        assert all(res.values()), (k.name, res)


def test_persistent_ring_schedule(built_lib):
    """The persistent kernels (128 x 128 tile, windows of 2, 4 and 8 K tiles): per
    K tile of the steady loop the MFMAs, copies and barrier of the ring plus
    16 / window stores, issued after the K tile's copies; one steady vmcnt wait
    of (S-2) x copies + (S-1) x stores, the kernel's other waits only the
    prologue's and the final drain; no spills or accumulator copies in the loop."""
    ks = X.load_persist()
    assert len(ks) == 8 * 8
    assert {(k.stages, k.window) for k in ks} == {(2, 2), (2, 4), (2, 8), (3, 2), (3, 4), (3, 8), (4, 4), (4, 8)}
    for k in ks:
        res = X.check_persist(k)
        assert all(res.values()), (k.name, res, X.persist_stats(k))


# ---- the checks see the mistakes the pages warn about ---------------------------------
def _planted(k, edits):
    """Copy of kernel k with instruction i's operation replaced by op, for each (i, op)."""
    import dataclasses
    ins = list(k.instrs)
    for i, op in edits:
        ins[i] = ins[i].split("|", 1)[0] + "|" + op
    return dataclasses.replace(k, instrs=ins)


def _ops(k):
    return [x.split("|", 1)[1] for x in k.instrs]


def _is_dma(op):
    return op.startswith("buffer_load") and op.rstrip().endswith("lds")


@pytest.mark.parametrize("tile,stages", [(4, 2), (1, 3)])
def test_checks_catch_planted_schedule_faults(kernels, tile, stages):
    """Each fault is planted in a copy of the shipped exact-fit DIRECT kernel's
    disassembly (on the CPU; no broken kernel is ever run): the steady loop's
    barrier removed; its vmcnt wait removed, loosened or tightened to 0 (an
    early wait); one copy dropped; the lgkmcnt(0) before the barrier loosened;
    a copy moved beside the barrier.  check() passes the real kernel and fails
    every planted one ("Pipeline GPU Kernel", Haeufige Stolperfallen: missing
    barriers, swapped commit/wait, a forgotten epilogue tile)."""
    (k,) = pick(kernels, dtype=0, bcol=False, tile=tile, variant="direct", stages=stages, exact=True)
    assert all(X.check(k).values())
    ops = _ops(k)
    bar = max(i for i, o in enumerate(ops) if o.startswith("s_barrier"))  # the steady loop's barrier
    vm = max(i for i in range(bar) if re.search(r"vmcnt\(\d+\)", ops[i]))
    lg = max(i for i in range(bar) if ops[i].startswith("s_waitcnt lgkmcnt(0)"))
    last_dma = max(i for i, o in enumerate(ops) if _is_dma(o))
    dma_after = min(i for i in range(bar + 1, len(ops)) if _is_dma(ops[i]))
    want = int(re.search(r"vmcnt\((\d+)\)", ops[vm]).group(1))
    planted = {
        "no barrier": ([(bar, "s_nop 0")], "counts"),
        "no wait": ([(vm, "s_nop 0")], "vmcnt"),
        "wait too loose": ([(vm, f"s_waitcnt vmcnt({want + 1})")], "vmcnt"),
        "copy dropped": ([(last_dma, "s_nop 0")], "counts"),
        "fragment reads not drained": ([(lg, "s_waitcnt lgkmcnt(1)")], "lgkmcnt"),
        "copy beside the barrier": ([(bar + 1, ops[dma_after]), (dma_after, ops[bar + 1])], "overlap"),
    }
    if want > 0:
        planted["early wait"] = ([(vm, "s_waitcnt vmcnt(0)")], "vmcnt")
    for name, (edits, prop) in planted.items():
        res = X.check(_planted(k, edits))
        assert not res[prop], (name, res)


def test_attention_checks_catch_planted_faults(built_lib):
    """Faults planted in copies of the shipped attention kernels (CPU only): DIRECT
    with its steady vmcnt wait removed, loosened or (3 stages) made a full drain,
    or a copy dropped; SYNC with its vmcnt(0) moved after the block's first MFMA;
    REG with its vmcnt(0) moved before the MFMAs that should overlap the loads."""
    ks = {(k.dtype, k.D, k.variant, k.stages): k for k in X.load_attention()}
    for st in (2, 3):
        k = ks[(0, 128, "direct", st)]
        assert all(X.check_attention(k).values())
        ops = _ops(k)
        body_start = X.steady_span(k)[0]
        vm = next(i for i in range(body_start, len(ops)) if re.search(r"vmcnt\(\d+\)", ops[i]))
        want = int(re.search(r"vmcnt\((\d+)\)", ops[vm]).group(1))
        dma = next(i for i in range(vm, len(ops)) if _is_dma(ops[i]))
        planted = {"no wait": [(vm, "s_nop 0")], "wait too loose": [(vm, f"s_waitcnt vmcnt({want + 1})")],
                   "copy dropped": [(dma, "s_nop 0")]}
        if want:
            planted["early wait"] = [(vm, "s_waitcnt vmcnt(0)")]
        for name, edits in planted.items():
            res = X.check_attention(_planted(k, edits))
            assert not all(res.values()), (st, name, res)
    for v, st in (("sync", 1), ("reg", 2)):
        k = ks[(0, 128, v, st)]
        assert all(X.check_attention(k).values())
        ops = _ops(k)
        start, end = X.steady_span(k)
        idx = range(start, end + 1)
        first_load = next(i for i in idx if ops[i].startswith("buffer_load"))
        wait = next(i for i in idx if i > first_load and re.search(r"vmcnt\(0\)", ops[i]))
        mfma_after = next(i for i in idx if i > first_load and ops[i].startswith("v_mfma"))
        if v == "sync":  # swap the drain with the first MFMA after the loads: compute overlaps them
            i, j = wait, next(i for i in idx if i > wait and ops[i].startswith("v_mfma"))
        else:  # move the drain up to right after the loads, before the MFMAs that overlap them
            i, j = wait, next(i for i in idx if i > max(x for x in idx if ops[x].startswith("buffer_load")))
        res = X.check_attention(_planted(k, [(i, ops[j]), (j, ops[i])]))
        assert not res["vmcnt"], (v, res, mfma_after)


# The kernels the library's own choice runs, and the exact-fit forms that the pipelining
# comparisons time (every (variant, stages) pair of a tile in the same form as its ring).
AUTO_CHOICES = {(1, "direct", 3), (2, "direct", 2), (3, "direct", 3), (3, "direct", 4), (4, "direct", 2),
                (6, "direct", 2)}
COMPARED = {("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2)}


def test_default_and_compared_kernels_keep_scratch_out_of_the_loop(kernels):
    """No scratch access in the steady loop of any kernel AUTO can select (the 256 x 256
    one-wave-per-SIMD tile only in its exact-fit form, as the planner selects it) or of the
    exact-fit forms the pipelining comparisons use.  Only the general int8 row-major-B
    8-wave kernel spills at all (2 registers, outside its loop)."""
    seen = 0
    for k in kernels:
        auto = (k.tile, k.variant, k.stages) in AUTO_CHOICES and (k.tile != 4 or k.exact)
        compared = k.exact and k.tile in (1, 2, 4, 5, 6) and (k.variant, k.stages) in COMPARED
        if not (auto or compared):
            continue
        seen += 1
        assert X.loop_stats(k)["scratch"] == 0, k.name
        if not (k.dtype == 2 and not k.bcol and k.tile == 2 and not k.exact):
            assert k.meta["vgpr_spill"] == 0 and k.meta["scratch"] == 0, (k.name, k.meta)
    # per table: 9 selectable (tiles 1, 2 and 6 in both forms, 3 general with 3 and 4 stages
    # (4: a row band), 4 exact) and 20 compared, 3 of them in both sets
    assert seen == 8 * (9 + 20 - 3)


def test_poison_build_writes_before_every_refill():
    """In the race-detection library (libspt_poison.so), every ring kernel's steady
    loop follows each barrier with one poison write per copy the wave will issue,
    then lgkmcnt(0), and only then the copies that refill the stage.  (So a read
    of that stage before its copies land meets the poison; see
    tests/test_poison_gpu.py.)"""
    from software_pipelined_tiling_amd import build as b
    if not os.path.exists(b.POISON_LIB):
        pytest.skip("libspt_poison.so not built")
    ks = [k for k in X.load(b.POISON_LIB) if k.variant == "direct"]
    assert len(ks) == 2 * 25  # the ring kernels of fp16 row-major B and int8 column-major B
    for k in ks:
        body = X.steady_loop(k)
        loads = k.geometry["loads_per_tile"]
        bars = [i for i, o in enumerate(body) if o.startswith("s_barrier")]
        assert len(bars) == k.geometry["tiles_per_iter"], k.name
        for b0 in bars:
            first_copy = next(i for i in range(b0, len(body)) if body[i].startswith("buffer_load")
                              and body[i].rstrip().endswith("lds"))
            seg = body[b0:first_copy]
            writes = [i for i, o in enumerate(seg) if o.startswith("ds_write")]
            assert len(writes) == loads, (k.name, len(writes), loads)
            assert any(o.startswith("s_waitcnt") and "lgkmcnt(0)" in o for o in seg[writes[-1]:]), k.name
