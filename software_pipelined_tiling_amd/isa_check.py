"""Disassembly checks of the built K-loop kernels (gfx950 code objects in libspt.so).

The pipelined loop only hides memory latency if the waits sit where the
schedule says they do; this module reads the machine code the library
actually ships and checks it, the counterpart of inspecting the SASS of a
cp.async pipeline ("Pipeline GPU Kernel", Schritt 4: verify that the loads
of the next tile are issued before the math of the current one and that the
wait comes only where its data is needed).

For each kernel it finds the steady-state loop (the backward branch whose
body holds the most MFMAs) and reports, per loop iteration:

  mfma, dma, global_loads, ds_reads, barriers   instruction counts
  vmcnt_waits / lgkmcnt_waits                  every s_waitcnt operand
  max_gap                                      the most non-MFMA instructions
                                               between two MFMAs
  scratch, acc_moves                           spill traffic and AGPR<->VGPR
                                               copies inside the loop
and from the code object's metadata the LDS size, VGPR/AGPR counts and spill
counts.  `check(kernel)` turns that into pass/fail properties:

  DIRECT ring (buffer_load ... lds into an S-stage ring):
    counts     MFMAs, copies and barriers per iteration match the plan
    vmcnt      one vmcnt wait per tile, each (S-2) x copies-per-tile: the
               copies of younger tiles stay in flight (for S >= 3 there is
               no vmcnt(0) in the steady state); a 3-stage ring run as 5
               half-stage slots keeps half a tile's copies in flight
               (copies-per-tile / 2)
    lgkmcnt    one lgkmcnt(0) per tile (before the barrier); every other
               lgkm wait is partial, so fragment reads overlap the MFMAs
    overlap    every copy sits in an MFMA gap of its own (none in the
               barrier's gap) and no gap holds more than 3 fragment reads:
               loads are interleaved with the MFMAs, not bunched
    clean      no scratch access and no accumulator copies in the loop
    lds        LDS size = S x stage bytes (2S - 1 half stages for such a ring)
  SYNC: the loop drains vmcnt(0) before its first MFMA (no overlap: the
  unpipelined reference).  REG: the tile's global loads are issued before the
  first MFMA of the iteration and their vmcnt wait comes after the last one.

The attention consumer's kernels are checked too (`check_attention`): per
key block the MFMAs of both products, DIRECT's copies, barrier and one
vmcnt((S-2) x copies) wait, REG's loads before the block's last MFMA and its
vmcnt(0) after it, SYNC's vmcnt(0) before its first MFMA, no scratch.

The streaming kernel (y = 2x, "Hiding Memory Latency ...", section 8) is
checked too (`check_stream`): per loop iteration one copy, one store and one
barrier, and the steady wait vmcnt(2S-3) (S >= 2: copies and stores share
the in-order counter; the S-1 younger copies and their stores stay in
flight); S = 1 waits for everything and has two barriers.

Command line:  python -m software_pipelined_tiling_amd.isa_check [name-regex]
"""
from __future__ import annotations

import dataclasses
import os
import re
import struct
import subprocess
import sys
import tempfile
from typing import Tuple, Dict, List, Optional

LLVM = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/llvm/bin")
HERE = os.path.dirname(os.path.abspath(__file__))

# Tile menu (BM, BN, K depth in bytes, waves along M, waves along N): the same
# values as kTiles in csrc/spt_config.h, restated to compute expected counts.
TILES = {1: (128, 256, 64, 2, 2), 2: (256, 256, 128, 2, 4), 3: (128, 128, 64, 2, 2),
         4: (256, 256, 128, 2, 2), 5: (256, 256, 64, 2, 2), 6: (256, 192, 128, 2, 4)}
ELT = {0: 2, 1: 2, 2: 1, 3: 4}
LDS_PER_CU = 163840
VARIANTS = {1: "sync", 2: "reg", 3: "direct"}
_CFG = re.compile(r"CfgILi(\d+)ELb(\d)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E")


@dataclasses.dataclass
class Kernel:
    name: str
    dtype: int
    bcol: bool
    tile: int
    variant: str
    stages: int
    exact: bool
    instrs: List[str]
    meta: Dict[str, int]

    # expected per-tile figures from the tile geometry
    @property
    def geometry(self):
        BM, BN, BKB, WM, WN = TILES[self.tile]
        waves = WM * WN
        fm, fn = BM // WM // 16, BN // WN // 16
        ks = BKB // 64
        mfma = fm * fn * ks * (4 if self.dtype == 3 else 1)
        loads = (BM * BKB + BKB * BN) // 16 // (64 * waves)
        stage = BM * BKB + BKB * BN
        # a DIRECT ring of S full stages that exceed the LDS, with A and B parts of one size,
        # runs as 2S - 1 half-stage slots; the copies of one half stay in flight per wait
        half = (self.variant == "direct" and self.stages * stage > LDS_PER_CU and BM == BN
                and (2 * self.stages - 1) * stage // 2 <= LDS_PER_CU)
        lds = (2 * self.stages - 1) * stage // 2 if half else self.stages * stage
        steady = (2 * self.stages - 5) * loads // 2 if half else (self.stages - 2) * loads
        return dict(mfma_per_tile=mfma, loads_per_tile=loads, ks=ks, stage_bytes=stage, lds_bytes=lds,
                    steady_vmcnt=steady, half_stage_slots=2 * self.stages - 1 if half else 0,
                    tiles_per_iter=1 if ks % 2 == 0 or self.variant != "direct" else 2)


def code_objects(lib: str) -> List[bytes]:
    """The gfx950 code objects of every offload bundle in the library's .hip_fatbin."""
    with tempfile.TemporaryDirectory() as td:
        fb = os.path.join(td, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}", lib,
                        os.path.join(td, "discard")], check=True, capture_output=True)
        data = open(fb, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out, i = [], data.find(magic)
    while i >= 0:
        n = struct.unpack_from("<Q", data, i + 24)[0]
        q = i + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", data, q)
            triple = data[q + 24:q + 24 + tl].decode()
            q += 24 + tl
            if triple.endswith("gfx950"):
                out.append(data[i + off:i + off + size])
        i = data.find(magic, i + 1)
    return out


def _disassemble(co: bytes) -> Dict[str, List[str]]:
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(co)
        f.flush()
        txt = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", f.name],
                             check=True, capture_output=True, text=True).stdout
    funcs: Dict[str, List[str]] = {}
    cur = None
    for line in txt.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur and line.startswith("\t"):
            body = line.strip()
            m2 = re.search(r"//\s*([0-9A-Fa-f]+):", body)
            addr = int(m2.group(1), 16) if m2 else -1
            funcs[cur].append(f"{addr:x}|" + body.split("//")[0].strip())
    return funcs


def _metadata(co: bytes) -> Dict[str, Dict[str, int]]:
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(co)
        f.flush()
        txt = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", f.name],
                             check=True, capture_output=True, text=True).stdout
    out: Dict[str, Dict[str, int]] = {}
    for block in txt.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        d = {"agpr": int(block.split("\n")[0])}
        for key, tag in (("lds", "group_segment_fixed_size"), ("scratch", "private_segment_fixed_size"),
                         ("vgpr", "vgpr_count"), ("sgpr", "sgpr_count"), ("vgpr_spill", "vgpr_spill_count"),
                         ("sgpr_spill", "sgpr_spill_count")):
            m = re.search(r"\." + tag + r":\s+(\d+)", block)
            d[key] = int(m.group(1)) if m else -1
        out[name.group(1)] = d
    return out


def load(lib: Optional[str] = None) -> List[Kernel]:
    lib = lib or os.path.join(HERE, "libspt.so")
    ks: List[Kernel] = []
    for co in code_objects(lib):
        meta = _metadata(co)
        for name, instrs in _disassemble(co).items():
            m = _CFG.search(name)
            if not m or "gemm_kernel" not in name:
                continue
            dt, bc, ti, v, s, ex, _bl = (int(x) for x in m.groups())
            ks.append(Kernel(name, dt, bool(bc), ti, VARIANTS[v], s, bool(ex), instrs, meta.get(name, {})))
    return ks


@dataclasses.dataclass
class PersistKernel(Kernel):
    window: int = 0  # K tiles over which the previous output tile is stored


_PERSIST = re.compile(r"gemm_persist_kernelI.*?EELi(\d+)EE")


def load_persist(lib: Optional[str] = None) -> List[PersistKernel]:
    """The persistent-workgroup kernels (csrc/spt_persist.hpp)."""
    lib = lib or os.path.join(HERE, "libspt.so")
    ks: List[PersistKernel] = []
    for co in code_objects(lib):
        meta = _metadata(co)
        for name, instrs in _disassemble(co).items():
            m, w = _CFG.search(name), _PERSIST.search(name)
            if not (m and w):
                continue
            dt, bc, ti, _v, s, ex, _bl = (int(x) for x in m.groups())
            ks.append(PersistKernel(name, dt, bool(bc), ti, "persist", s, bool(ex), instrs,
                                    meta.get(name, {}), int(w.group(1))))
    return ks


def persist_stats(k: PersistKernel) -> dict:
    """Figures of the steady loop of a persistent kernel: the shortest loop body
    holding the MFMAs of two K tiles (the loop past the store window), plus
    every vmcnt wait of the whole kernel."""
    g = k.geometry
    bodies = [b for b in loop_regions(k) if _count_mfma(b) == 2 * g["mfma_per_tile"]]
    body = min(bodies, key=len) if bodies else []
    vm_all = [int(m.group(1)) for x in k.instrs for m in [re.search(r"vmcnt\((\d+)\)", _op(x))] if m]
    # copies before stores within every K tile: split the body (read as a cycle) at its barriers
    order_ok = bool(body)
    if body and any(x.startswith("s_barrier") for x in body):
        b0 = next(i for i, x in enumerate(body) if x.startswith("s_barrier"))
        rot = body[b0:] + body[:b0]
        seg: List[str] = []
        segs: List[List[str]] = []
        for x in rot:
            if x.startswith("s_barrier") and seg:
                segs.append(seg)
                seg = []
            seg.append(x)
        segs.append(seg)
        for sg in segs:
            cp = [i for i, x in enumerate(sg) if x.startswith("buffer_load") and x.rstrip().endswith("lds")]
            st = [i for i, x in enumerate(sg) if x.startswith("buffer_store")]
            if cp and st and max(cp) > min(st):
                order_ok = False
    return dict(
        instructions=len(body), mfma=_count_mfma(body), dma=_count_copies(body),
        stores=sum(x.startswith("buffer_store") for x in body),
        barriers=sum(x.startswith("s_barrier") for x in body),
        vmcnt_waits=[int(m.group(1)) for x in body for m in [re.search(r"vmcnt\((\d+)\)", x)] if m],
        kernel_vmcnt_waits=sorted(set(vm_all)),
        scratch=sum(x.startswith("scratch_") for x in body),
        acc_moves=sum(x.startswith("v_accvgpr") for x in body),
        copies_before_stores=order_ok,
    )


def check_persist(k: PersistKernel) -> Dict[str, bool]:
    """The persistent kernel's schedule: per K tile of its steady loop the MFMAs,
    copies and one barrier of the ring plus (wave-tile blocks) / window stores, issued after the
    copies; one steady vmcnt wait, (S-2) x copies + (S-1) x stores per K tile;
    the kernel's other waits only the prologue's and the final drain; no spills
    or accumulator copies in the loop; the LDS ring of S stages."""
    g, st = k.geometry, persist_stats(k)
    BM, BN, _bkb, WM, WN = TILES[k.tile]
    S, L, ST = k.stages, g["loads_per_tile"], (BM // WM // 16) * (BN // WN // 16) // k.window
    steady = (S - 2) * L + (S - 1) * ST
    first = (S - 1) * L + S * ST
    return {
        "counts": (st["mfma"] == 2 * g["mfma_per_tile"] and st["dma"] == 2 * L and st["stores"] == 2 * ST
                   and st["barriers"] == 2),
        "vmcnt": len(st["vmcnt_waits"]) == 2 and all(v == steady for v in st["vmcnt_waits"]),
        "kernel_vmcnt": set(st["kernel_vmcnt_waits"]) <= {steady, first, 0},
        "order": st["copies_before_stores"],
        "clean": st["scratch"] == 0 and st["acc_moves"] == 0,
        "lds": k.meta.get("lds") == S * g["stage_bytes"],
    }


@dataclasses.dataclass
class StreamKernel:
    name: str
    stages: int
    instrs: List[str]
    meta: Dict[str, int]


def load_stream(lib: Optional[str] = None) -> List[StreamKernel]:
    lib = lib or os.path.join(HERE, "libspt.so")
    out: List[StreamKernel] = []
    for co in code_objects(lib):
        meta = _metadata(co)
        for name, instrs in _disassemble(co).items():
            m = re.search(r"scale_by_two_kernelILi(\d+)E", name)
            if m:
                out.append(StreamKernel(name, int(m.group(1)), instrs, meta.get(name, {})))
    return out


def check_stream(k: StreamKernel) -> Dict[str, bool]:
    # the ring loop: the shortest loop body that holds a copy and a barrier
    cands = [b for b in loop_regions(k) if _count_copies(b) and any(x.startswith("s_barrier") for x in b)]
    body = min(cands, key=len) if cands else []
    dma = sum(x.startswith("buffer_load") and x.rstrip().endswith("lds") for x in body)
    st = sum(x.startswith("buffer_store") for x in body)
    bar = sum(x.startswith("s_barrier") for x in body)
    vm = [int(m.group(1)) for x in body for m in [re.search(r"vmcnt\((\d+)\)", x)] if m]
    S = k.stages
    res = {"counts": dma == 1 and st == 1 and bar == (2 if S == 1 else 1),
           "vmcnt": vm == ([0] if S == 1 else [2 * S - 3]),
           "lds": k.meta.get("lds") == S * 4096,
           "clean": not any(x.startswith("scratch_") for x in body)}
    return res


@dataclasses.dataclass
class AttnKernel:
    name: str
    dtype: int
    D: int
    variant: str
    stages: int
    instrs: List[str]
    meta: Dict[str, int]

    @property
    def geometry(self):
        """Per key block: BKV keys, MFMAs per wave (S = Q K^T, O += P V and the row sums
        of P over the wave's 64 query rows), 16-byte copies per thread, stage bytes (K
        and V blocks)."""
        bkv = 32 if self.D == 128 else 64
        fm = 2  # 16-row query blocks per wave (32 rows; 8 waves, two per SIMD)
        mfma = fm * (bkv // 16) * (self.D // 32) + fm * (self.D // 16) * (bkv // 32) + fm * (bkv // 32)
        loads = 2 * (bkv * self.D * 2) // 16 // 512
        return dict(bkv=bkv, mfma_per_block=mfma, loads_per_block=loads, stage_bytes=2 * bkv * self.D * 2)


_ATTN = re.compile(r"AttnCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")


def load_attention(lib: Optional[str] = None) -> List[AttnKernel]:
    """The attention consumer's kernels (csrc/spt_attention.hip)."""
    lib = lib or os.path.join(HERE, "libspt.so")
    out: List[AttnKernel] = []
    for co in code_objects(lib):
        meta = _metadata(co)
        for name, instrs in _disassemble(co).items():
            m = _ATTN.search(name)
            if m and "attention_kernel" in name:
                dt, d, v, s = (int(x) for x in m.groups())
                out.append(AttnKernel(name, dt, d, VARIANTS[v], s, instrs, meta.get(name, {})))
    return out


def check_attention(k: AttnKernel) -> Dict[str, bool]:
    """The key/value block loop of an attention kernel (the loop body holding the
    most MFMAs), which holds U blocks: one turn of the ring for DIRECT (U = S) and
    for the two-stage REG (U = 2), unrolled so that each block's stage is a
    constant, else one block.  Per block its MFMAs; DIRECT: its copies, one barrier
    and one vmcnt wait of (S-2) x copies, so the copies of the S-2 younger blocks
    stay in flight; REG: the block's global loads, each followed by MFMAs before
    the vmcnt(0) that waits for it; SYNC: vmcnt(0) before the first MFMA; no
    scratch anywhere; no accumulator-register copies in the loop (the MFMAs write
    VGPRs, where the softmax reads them); the LDS ring of S stages."""
    g = k.geometry
    body = steady_loop(k)
    L, S = g["loads_per_block"], k.stages
    U = S if k.variant == "direct" else 2 if (k.variant == "reg" and S == 2) else 1
    loads = [i for i, x in enumerate(body) if x.startswith("buffer_load") and not x.rstrip().endswith("lds")]
    if loads:  # read the loop as a cycle starting at its first global load
        body = body[loads[0]:] + body[:loads[0]]
        loads = [i for i, x in enumerate(body) if x.startswith("buffer_load") and not x.rstrip().endswith("lds")]
    mf = [i for i, x in enumerate(body) if x.startswith("v_mfma")]
    vm = [(i, int(m.group(1))) for i, x in enumerate(body) for m in [re.search(r"vmcnt\((\d+)\)", x)] if m]
    bar = sum(x.startswith("s_barrier") for x in body)
    res = {"counts": _count_mfma(body) == U * g["mfma_per_block"],
           "clean": k.meta.get("scratch") == 0 and not any(x.startswith("scratch_") for x in body),
           "vgpr_form": not any(x.startswith("v_accvgpr_") for x in body),
           "lds": k.meta.get("lds") == S * g["stage_bytes"]}
    if k.variant == "direct":
        res["copies"] = _count_copies(body) == U * L and bar == U
        res["vmcnt"] = [v for _, v in vm] == [(S - 2) * L] * U
    elif k.variant == "reg":
        # after each load, MFMAs before the first wait, which is vmcnt(0) (the compiler adds its
        # own, already satisfied, partial waits before each staged ds_write)
        res["copies"] = len(loads) == U * L and bar == U * (2 if S == 1 else 1)
        ok = bool(vm)
        for li in loads:
            w = next((wi for wi, _ in vm if wi > li), None)
            if w is None:
                ok = False
                break
            last = max(x for x in loads if x < w)
            ok = ok and dict(vm)[w] == 0 and any(last < m < w for m in mf)
        res["vmcnt"] = ok
    else:
        # from the loads on: vmcnt(0) before any MFMA
        res["copies"] = len(loads) == L and bar == 2
        res["vmcnt"] = bool(mf) and bool(vm) and vm[0][1] == 0 and vm[0][0] < mf[0]
    return res


def _op(ins: str) -> str:
    return ins.split("|", 1)[1]


def _count_mfma(body: List[str]) -> int:
    return sum(x.startswith("v_mfma") for x in body)


def _count_copies(body: List[str]) -> int:
    return sum(x.startswith("buffer_load") and x.rstrip().endswith("lds") for x in body)


def loop_spans(k) -> List[Tuple[int, int]]:
    """(first, last) indices into k.instrs of every loop body: from the target of a
    backward branch to the branch, as laid out."""
    addr = [int(i.split("|")[0], 16) for i in k.instrs]
    pos = {a: n for n, a in enumerate(addr)}
    out: List[Tuple[int, int]] = []
    for j, ins in enumerate(k.instrs):
        m2 = re.match(r"s_c?branch\w*\s+(\d+)$", _op(ins))
        if not m2:
            continue
        simm = int(m2.group(1))  # signed 16-bit target in dwords, relative to the next instruction
        simm = simm - 65536 if simm >= 32768 else simm
        nxt = addr[j + 1] if j + 1 < len(addr) else addr[j] + 4
        tgt = nxt + 4 * simm
        if tgt <= addr[j] and tgt in pos:
            out.append((pos[tgt], j))
    return out


def loop_regions(k) -> List[List[str]]:
    """Instructions from the target of every backward branch to the branch
    (the body of a loop, as laid out)."""
    return [[_op(x) for x in k.instrs[a:b + 1]] for a, b in loop_spans(k)]


def steady_span(k, key=None) -> Tuple[int, int]:
    """(first, last) indices into k.instrs of the loop that steady_loop returns."""
    key = key or _count_mfma
    best, bs = None, []
    for a, b in loop_spans(k):
        body = [_op(x) for x in k.instrs[a:b + 1]]
        if best is None or key(body) > key(bs) or (key(body) == key(bs) > 0 and len(body) < len(bs)):
            best, bs = (a, b), body
    return best


def steady_loop(k, key=_count_mfma) -> List[str]:
    """The loop body holding the most MFMAs (or the most of what `key` counts);
    among equals the shortest."""
    best: List[str] = []
    for body in loop_regions(k):
        if key(body) > key(best) or (key(body) == key(best) > 0 and len(body) < len(best)):
            best = body
    return best


def cyclic_gaps(body: List[str]) -> List[List[str]]:
    """The non-MFMA instructions between consecutive MFMAs of a loop body, the
    gap across the back edge included (the body read as a cycle)."""
    mf = [i for i, x in enumerate(body) if x.startswith("v_mfma")]
    if not mf:
        return []
    rot = body[mf[0]:] + body[:mf[0]]  # starts with an MFMA
    gaps: List[List[str]] = []
    cur: List[str] = []
    for x in rot[1:]:
        if x.startswith("v_mfma"):
            gaps.append(cur)
            cur = []
        else:
            cur.append(x)
    gaps.append(cur)  # the gap across the back edge, before the first MFMA
    return gaps


def loop_stats(k: Kernel) -> dict:
    body = steady_loop(k)
    mf = [i for i, x in enumerate(body) if x.startswith("v_mfma")]
    cg = cyclic_gaps(body)
    gaps = [len(g) for g in cg]
    between = lambda pred: sum(1 for i, x in enumerate(body) if pred(x) and mf and mf[0] < i < mf[-1])
    is_dma = lambda x: x.startswith("buffer_load") and x.rstrip().endswith("lds")
    is_gld = lambda x: x.startswith("buffer_load") and not x.rstrip().endswith("lds")
    is_dsr = lambda x: x.startswith("ds_read")
    waits = [x for x in body if x.startswith("s_waitcnt")]
    vm = [int(m.group(1)) for x in waits for m in [re.search(r"vmcnt\((\d+)\)", x)] if m]
    lg = [int(m.group(1)) for x in waits for m in [re.search(r"lgkmcnt\((\d+)\)", x)] if m]
    first_mfma = mf[0] if mf else 0
    last_mfma = mf[-1] if mf else 0
    return dict(
        instructions=len(body), mfma=len(mf),
        dma=sum(map(is_dma, body)), dma_between_mfma=between(is_dma),
        global_loads=sum(map(is_gld, body)), global_loads_before_first_mfma=sum(
            1 for i, x in enumerate(body) if is_gld(x) and i < first_mfma),
        ds_reads=sum(map(is_dsr, body)), ds_reads_between_mfma=between(is_dsr),
        barriers=sum(x.startswith("s_barrier") for x in body),
        vmcnt_waits=vm, lgkmcnt_waits=lg,
        vmcnt0_before_first_mfma=any(re.search(r"vmcnt\(0\)", x) for x in body[:first_mfma]),
        vmcnt_after_last_mfma=[int(m.group(1)) for x in body[last_mfma:] for m in [re.search(r"vmcnt\((\d+)\)", x)] if m],
        max_gap=max(gaps) if gaps else 0, mean_gap=round(sum(gaps) / len(gaps), 2) if gaps else 0.0,
        dma_per_gap_max=max((sum(map(is_dma, g)) for g in cg), default=0),
        ds_reads_per_gap_max=max((sum(map(is_dsr, g)) for g in cg), default=0),
        dma_in_barrier_gap=sum(sum(map(is_dma, g)) for g in cg if any(x.startswith("s_barrier") for x in g)),
        scratch=sum(x.startswith("scratch_") for x in body),
        acc_moves=sum(x.startswith("v_accvgpr") for x in body),
    )


def check(k: Kernel) -> Dict[str, bool]:
    """Pass / fail of the properties in the module docstring."""
    g, st = k.geometry, loop_stats(k)
    T = g["tiles_per_iter"]
    res: Dict[str, bool] = {}
    if k.variant == "direct":
        res["counts"] = (st["mfma"] == T * g["mfma_per_tile"] and st["dma"] == T * g["loads_per_tile"]
                         and st["barriers"] == T)
        res["vmcnt"] = len(st["vmcnt_waits"]) == T and all(v == g["steady_vmcnt"] for v in st["vmcnt_waits"])
        res["lgkmcnt"] = st["lgkmcnt_waits"].count(0) == T
        # each copy in an MFMA gap of its own, none in the gap of the barrier, fragment
        # reads at most 3 to a gap (a 16-cycle MFMA leaves about three issue slots)
        res["overlap"] = (st["dma_per_gap_max"] == 1 and st["dma_in_barrier_gap"] == 0
                          and st["ds_reads_per_gap_max"] <= 3)
        res["clean"] = st["scratch"] == 0 and st["acc_moves"] == 0
        res["lds"] = k.meta.get("lds") == g["lds_bytes"]
    elif k.variant == "sync":
        res["no_overlap"] = st["vmcnt0_before_first_mfma"]
        res["lds"] = k.meta.get("lds") == g["stage_bytes"]
    else:  # reg
        res["loads_ahead"] = st["global_loads_before_first_mfma"] == st["global_loads"] > 0
        res["wait_after_mfma"] = 0 in st["vmcnt_after_last_mfma"]
        res["lds"] = k.meta.get("lds") == k.stages * g["stage_bytes"]
    return res


def report(pattern: str = ".", lib: Optional[str] = None) -> List[dict]:
    rows = []
    for k in load(lib):
        if not re.search(pattern, k.name):
            continue
        rows.append(dict(kernel=k.name, dtype=k.dtype, bcol=k.bcol, tile=k.tile, variant=k.variant,
                         stages=k.stages, exact=k.exact, meta=k.meta, loop=loop_stats(k), checks=check(k)))
    return rows


if __name__ == "__main__":
    import json
    for r in report(sys.argv[1] if len(sys.argv) > 1 else "."):
        print(json.dumps(r))
