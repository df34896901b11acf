"""The planning-formula oracle against the pages' own worked numbers (no GPU)."""
import json
import os

import pytest

from oracle import plan_oracle as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")
KB = 1024


@pytest.fixture(scope="module")
def nums():
    with open(os.path.join(GOLD, "pages_planner_numbers.json")) as f:
        return json.load(f)


def test_stage_and_ring_bytes(nums):
    t = nums["tile_128x256x32_fp16"]
    assert t["BM"] * t["BK"] * t["elt"] == t["a_stage_bytes"]
    assert P.stage_bytes(t["BM"], t["BN"], t["BK"], t["elt"]) == t["stage_bytes"]
    assert P.ring_bytes(t["BM"], t["BN"], t["BK"], t["elt"], 3) == t["ring_bytes_3"]
    assert (P.ring_bytes(t["BM"], t["BN"], t["BK"], t["elt"], 4)
            - P.ring_bytes(t["BM"], t["BN"], t["BK"], t["elt"], 3)) == t["extra_bytes_per_stage"]


def test_copy_decomposition(nums):
    t = nums["tile_128x256x32_fp16"]
    assert P.copies_per_thread(t["BM"], t["BK"], t["elt"], t["threads"], t["copy_bytes"]) == \
        t["a_copies_per_thread"]
    assert P.copies_per_thread(t["BK"], t["BN"], t["elt"], t["threads"], t["copy_bytes"]) == \
        t["b_copies_per_thread"]


def test_double_buffer_example(nums):
    d = nums["double_buffer_example"]
    # 32 x 32 half tiles give the 2 KB + 2 KB of the example
    assert P.stage_bytes(32, 32, 32, 2) == d["single_bytes"]
    assert P.ring_bytes(32, 32, 32, 2, 2) == d["double_bytes"]


def test_ga104_occupancy_cliff(nums):
    g = nums["ga104_limits"]
    m = P.Machine(g["regs_per_sm"], g["smem_per_sm_kb"] * KB, g["max_warps_per_sm"],
                  g["max_blocks_per_sm"], g["warp_size"])
    for kb, blocks in nums["ga104_cliff_cases"]["blocks_at_kb"].items():
        b, warps, lim = P.occupancy(m, 32, int(kb) * KB, 128)
        assert b == blocks and lim["smem"] == blocks, (kb, lim)
        assert warps == 4 * blocks  # 128 threads = 4 warps per block
    cliff = g["smem_per_sm_kb"] // 2
    assert cliff == g["cliff_kb"]
    for kb in nums["ga104_cliff_cases"]["doubled_over_cliff_from_kb"]:
        assert 2 * kb > cliff
        assert P.occupancy(m, 32, 2 * kb * KB, 128)[0] == 1


def test_occupancy_takes_the_minimum():
    m = P.Machine(65536, 100 * KB, 48, 16, 32)
    # 255 registers x 256 threads: register-limited to one block
    b, _, lim = P.occupancy(m, 255, 1 * KB, 256)
    assert b == 1 and lim["registers"] == 1
    # 16 warps per block: warp-limited to three blocks
    b, _, lim = P.occupancy(m, 16, 1 * KB, 512)
    assert b == 3 and lim["warps"] == 3


def test_balance_points(nums):
    g = nums["ga104_balance_points"]
    assert round(P.balance_point(g["fp32_gflops"], g["dram_gbs"]), 1) == g["fp32"]
    assert round(P.balance_point(g["fp16_tc_gflops"], g["dram_gbs"]), 1) == g["fp16_tc"]
    assert round(P.balance_point(g["int8_tc_gops"], g["dram_gbs"]), 1) == g["int8_tc"]


def test_ratio_closed_form():
    # 2*BM*BN*BK / ((BM*BK + BK*BN) * elt) == 2*BM*BN / ((BM+BN)*elt): square tiles give B/elt
    for b, elt in [(64, 2), (128, 2), (256, 1), (32, 4)]:
        assert P.compute_load_ratio(b, b, 32, elt) == b / elt
    assert P.compute_load_ratio(128, 256, 32, 2) == pytest.approx(2 * 128 * 256 / (384 * 2))


def _read_schedule():
    pro, steady, stagemap = [], [], {}
    with open(os.path.join(GOLD, "ring_schedule_s3.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            if p[0] == "prologue":
                pro.append((int(p[4]), int(p[5])))
            elif p[0] == "steady":
                steady.append(tuple(int(x) for x in p[1:]))
            else:
                stagemap[int(p[1][1:])] = int(p[2])
    return pro, steady, stagemap


def test_ring_schedule_matches_pages_table():
    pro, steady, stagemap = _read_schedule()
    got_pro, got_steady = P.ring_schedule(3, 8)
    assert got_pro == pro
    assert [tuple(r) for r in got_steady[: len(steady)]] == steady
    for tile, stage in stagemap.items():
        assert got_steady[tile][2] == stage


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("nt", [1, 2, 3, 5, 9])
def test_ring_invariants(S, nt):
    """Producer never overwrites an in-use stage; consumer never reads an unissued tile."""
    pro, steady = P.ring_schedule(S, nt)
    issued = {t: s for t, s in pro}
    occupant = {s: t for t, s in pro}
    for it, ct, cs, ft, fs in steady:
        if ft is not None:
            # the issued stage is not the one consumed now (unless S == 1, the synchronous loop)
            assert S == 1 or fs != cs
            # whatever the stage held has already been consumed
            assert occupant.get(fs, -1) < ct or (S == 1 and occupant.get(fs, -1) == ct - 1)
            issued[ft] = fs
            occupant[fs] = ft
        assert issued.get(ct) == cs and occupant[cs] == ct  # consumed tile is the stage's occupant
    assert sorted(issued) == list(range(nt))
