"""Plain restatement of the pages' planning formulas (test infrastructure only).

TEST INFRASTRUCTURE ONLY: used by the test-suite to check the integer planning
figures that the HIP library's planner reports.  It imports nothing from the
library.  Every function is one formula from the pages, in their notation:

* ``stage_bytes``   -- "Pipeline GPU Kernel", Schritt 1: smem_a_size =
  BM*BK*sizeof(T), smem_b_size = BK*BN*sizeof(T); one pipeline stage holds both
  (also "Hiding Memory Latency ...", section 6, "one K stage").
* ``ring_bytes``    -- the ring holds ``stages`` such stages ("Hiding Memory
  Latency ...", sections 5, 6 and 10).
* ``compute_load_ratio`` -- "Pipeline GPU Kernel", Schritt 2: 2*BM*BN*BK /
  ((BM*BK + BK*BN) * sizeof(T)), FLOP per loaded byte of one tile.
* ``copies_per_thread`` -- "Hiding Memory Latency ...", section 6: a stage is
  moved by THREADS threads in 16-byte accesses, tile_bytes / (THREADS * 16)
  per thread.
* ``occupancy``     -- "Kernel-Engpass analysieren", Schritt 3: resident
  blocks = min(register limit, shared-memory limit, warp limit, block limit).
* ``balance_point`` -- "Kernel-Engpass analysieren", Schritt 2: peak compute /
  peak bandwidth, in FLOP per byte.
* ``ring_schedule`` -- "Hiding Memory Latency ...", sections 5, 8 and 9: the
  prologue issues tiles 0..S-2 into stages 0..S-2; iteration t consumes tile t
  from stage t mod S and issues tile t+S-1 into stage (t+S-1) mod S.
"""
from __future__ import annotations

from dataclasses import dataclass


def stage_bytes(BM: int, BN: int, BK: int, elt: int) -> int:
    return BM * BK * elt + BK * BN * elt


def ring_bytes(BM: int, BN: int, BK: int, elt: int, stages: int) -> int:
    return stages * stage_bytes(BM, BN, BK, elt)


def compute_load_ratio(BM: int, BN: int, BK: int, elt: int) -> float:
    return (2 * BM * BN * BK) / ((BM * BK + BK * BN) * elt)


def copies_per_thread(rows: int, cols: int, elt: int, threads: int, vec_bytes: int = 16) -> float:
    return rows * cols * elt / (threads * vec_bytes)


@dataclass(frozen=True)
class Machine:
    """Per-multiprocessor limits used by the occupancy formula."""
    regs_per_sm: int        # 32-bit registers in one SM / CU
    smem_per_sm: int        # bytes of shared memory / LDS in one SM / CU
    max_warps_per_sm: int   # resident warps / waves
    max_blocks_per_sm: int  # resident blocks / workgroups
    warp_size: int


def occupancy(m: Machine, regs_per_thread: int, smem_per_block: int, threads_per_block: int):
    """Blocks per SM = min of the four limits; returns (blocks, active warps, limits dict)."""
    warps_per_block = -(-threads_per_block // m.warp_size)
    limits = {
        "registers": (m.regs_per_sm // (regs_per_thread * threads_per_block)
                      if regs_per_thread > 0 else m.max_blocks_per_sm),
        "smem": m.smem_per_sm // smem_per_block if smem_per_block > 0 else m.max_blocks_per_sm,
        "warps": m.max_warps_per_sm // warps_per_block,
        "blocks": m.max_blocks_per_sm,
    }
    blocks = min(limits.values())
    return blocks, blocks * warps_per_block, limits


def balance_point(peak_flops: float, bytes_per_s: float) -> float:
    return peak_flops / bytes_per_s


def ring_schedule(stages: int, num_tiles: int):
    """Return (prologue, steady) for an S-stage ring.

    prologue: list of (tile, stage) issued before the first consume.
    steady:   list of (iteration, consume_tile, consume_stage, issue_tile, issue_stage);
              issue_tile is None once the tiles run out (the epilogue drains).
    """
    prologue = [(t, t % stages) for t in range(min(stages - 1, num_tiles))]
    steady = []
    for t in range(num_tiles):
        fut = t + stages - 1
        steady.append((t, t, t % stages, fut if fut < num_tiles else None,
                       fut % stages if fut < num_tiles else None))
    return prologue, steady
