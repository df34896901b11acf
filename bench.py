#!/usr/bin/env python3
"""Benchmark of the software-pipelined GEMM K-loop on one MI355X.

One step = one C = A*B call of the library on the headline workload (fp16
GEMM 4096x4096x4096, A and B row-major, fp32 accumulation and fp32 C, entries
uniform in [-1, 1] rounded to fp16 from a fixed seed), inputs resident in HBM
before the timed region.  Prints ONE JSON line.

Besides the headline value it reports, in the same line:
  roofline      the dominant (only) kernel's achieved TFLOP/s against the
                dense fp16 MFMA peak, timed with HIP events on the stream
                the kernel runs on; HBM traffic from rocprofv3 counters when
                a summary taken on the current kernel source is committed
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  sweep         every (tile, variant, stages) of the library on the
                headline workload, the unpipelined one included
  workloads     int8 4096^3 (B column-major), bf16 8192^2 x K low-K sweep
                (with HBM GB/s), bf16 4000x3000x1000 ragged, fp16 256^3
  attention     the attention-style consumer (flash-attention forward, fp16,
                32 x 4096 x 4096 x 128) under every producer, and the ratio of
                register-staged to direct-to-LDS time (the pages' high-ratio claim)
  streaming     y = 2x through the S-stage ring: the pages' demonstration
                (2^20 floats, one block, 3 stages) and 2^28 floats over many
                blocks, each with the unpipelined S = 1 loop beside it
  power         socket power and GFX clocks sampled with amd-smi while the
                headline kernel runs back to back for a few seconds, and the
                dense peak at that clock (context for the roofline fraction)
  mfma_ceiling  the rate MFMAs alone sustain with the headline's operand data
                under the power limit (spt_probe_mfma in libspt_probe.so, built from
                bench_probe.hip), and value / that rate
  vendor_hipblaslt  the vendor library (torch.mm with fp32 output, torch._int_mm
                for int8) on the same operands, per workload too (context only)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "i8": 5033.2, "f32": 157.3}  # dense MFMA, MI355X
HBM_GBS = 8000.0
PAIRS = [("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2), ("direct", 3), ("direct", 4)]
TILES = (1, 2, 3, 4, 5, 6)
FLOP_PER_CLK = {"f16": 256 * 4096, "bf16": 256 * 4096, "i8": 256 * 8192}  # dense MFMA, whole chip


# The sources that define the headline's GEMM kernel (its template, tile menu,
# instantiation and translation unit): a committed counter summary applies
# only while these are unchanged.
KERNEL_SOURCES = ("spt_kernel.hpp", "spt_config.h", "spt_instances.hpp", "spt_registry.h", "spt_kernels_f16_row.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiling_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def to_dev(x: np.ndarray, dtype: str):
    import torch
    if dtype in ("f16", "bf16"):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy())
        return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).copy()).cuda()


class Problem:
    """Device-resident operands and output of one workload."""

    def __init__(self, w):
        import torch
        from software_pipelined_tiling_amd import inputs as I
        self.w = w
        self.A, self.B = I.make_operands(w)
        self.dA, self.dB = to_dev(self.A, w.dtype), to_dev(self.B, w.dtype)
        self.C = torch.empty((w.M, w.N), dtype=torch.int32 if w.dtype == "i8" else torch.float32,
                             device="cuda")

    def args(self, stream, variant="auto", stages=0, tile=0):
        import software_pipelined_tiling_amd as spt
        w = self.w
        return (w.M, w.N, w.K, self.dA.data_ptr(), self.A.shape[1], self.dB.data_ptr(),
                self.B.shape[1], self.C.data_ptr(), w.N, spt.DTYPE_CODES[w.dtype], stream,
                spt.COL if w.b_col else spt.ROW, spt.VARIANT_CODES[variant], stages, tile)


def vendor_us(prob: Problem, steps: int = 20):
    """Microseconds per call of the vendor library (hipBLASLt through torch) on the same
    device operands and the same output type: torch.mm(..., out_dtype=float32) for
    fp16/bf16, torch._int_mm for int8, timed like the library (time_graph).  Context
    only; None where torch has no such call."""
    import torch
    w = prob.w
    a = prob.dA[:, :w.K]
    b = prob.dB[:, :w.K].t() if w.b_col else prob.dB[:w.K, :w.N]
    if w.dtype == "i8":
        fn = lambda: torch._int_mm(a, b)
    elif w.dtype in ("f16", "bf16"):
        fn = lambda: torch.mm(a, b, out_dtype=torch.float32)
    else:
        return None
    try:
        for _ in range(3):
            fn()
        us = time_graph(lambda stream: fn() is not None, calls=steps)
        return None if us is None else round(us, 2)
    except Exception:  # shape or type torch does not support, or not capturable
        return None


def c_store_only(prob: Problem):
    """Microseconds per call of the plan the library picks for `prob`, run with K = 0:
    the kernel then only writes C (zeros), the floor under the C store of that plan."""
    import software_pipelined_tiling_amd as spt
    w = prob.w
    rc, pi = spt.spt_plan(spt.DTYPE_CODES[w.dtype], w.M, w.N, w.K, spt.COL if w.b_col else spt.ROW)
    if rc != 0:
        return None
    vname = {1: "sync", 2: "reg", 3: "direct", 4: "persist"}[pi.variant]
    return gemm_us(prob, vname, pi.stages, pi.tile_id, K=0)


def time_calls(prob: Problem, steps: int, warmup: int, variant="auto", stages=0, tile=0):
    """Mean ms per call over `steps` back-to-back calls, HIP events on the launch stream."""
    import torch
    import software_pipelined_tiling_amd as spt
    stream = torch.cuda.current_stream()
    a = prob.args(stream.cuda_stream, variant, stages, tile)
    rc = spt.spt_gemm_ex(*a)
    if rc != 0:
        return None
    for _ in range(warmup):
        spt.spt_gemm_ex(*a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        spt.spt_gemm_ex(*a)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_graph(fn, calls: int = 20, reps: int = 10, settle_s: float = 0.02):
    """Microseconds per call of `fn(stream_handle)` with `calls` calls captured in one
    HIP graph: the graph is replayed untimed for `settle_s` seconds (the clock settles
    after the previous workload), then `reps` times with an event pair around each
    replay; the median replay over `calls`.  This is the GPU time of back-to-back
    calls, host launch cost excluded (short kernels launched one by one from Python
    would wait on the host)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        if fn(side.cuda_stream) is False:  # eager check (and warm-up) before capture
            return None
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for _ in range(calls):
                fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < 1 or time.perf_counter() - t0 < settle_s:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    del g
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return per[len(per) // 2] / calls * 1e3


def gemm_us(prob: Problem, variant="auto", stages=0, tile=0, K=None):
    """time_graph of one spt_gemm_ex configuration (None when the library refuses it)."""
    import software_pipelined_tiling_amd as spt

    def fn(stream):
        a = list(prob.args(stream, variant, stages, tile))
        if K is not None:
            a[2] = K
        return spt.spt_gemm_ex(*a) == 0
    us = time_graph(fn)
    return None if us is None else round(us, 2)


def preheat(prob: Problem, seconds: float, variant="auto", stages=0, tile=0):
    """Run the call back to back, untimed, for `seconds` of wall time, so that the
    timed region starts with the GPU past its idle state and its clock settled
    under the power limit (a fresh GPU ramps for tens of ms).  Returns the calls made."""
    import torch
    import software_pipelined_tiling_amd as spt
    a = prob.args(torch.cuda.current_stream().cuda_stream, variant, stages, tile)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(100):
            spt.spt_gemm_ex(*a)
        torch.cuda.synchronize()
        n += 100
    return n


def time_calls_each(prob: Problem, steps: int, warmup: int, variant="auto", stages=0, tile=0):
    """`steps` back-to-back calls with a HIP event recorded on the launch stream
    before the first call and after every call: (mean ms per call over the whole
    region, list of per-call microseconds)."""
    import torch
    import software_pipelined_tiling_amd as spt
    stream = torch.cuda.current_stream()
    a = prob.args(stream.cuda_stream, variant, stages, tile)
    for _ in range(warmup):
        spt.spt_gemm_ex(*a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        spt.spt_gemm_ex(*a)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def cpu_baseline(w, budget_s: float):
    """The CPU oracle (as it stands) on the first rows of the same workload."""
    from oracle import oracle as O
    from software_pipelined_tiling_amd import inputs as I
    A, B = I.make_operands(w)
    cores = O.max_threads()
    # calibrate on 128 rows, then one measured run sized to the budget (capped at all rows)
    t0 = time.perf_counter()
    O.gemm(np.ascontiguousarray(A[:128]), B, w.dtype, b_col=w.b_col)
    rate = 128 / max(time.perf_counter() - t0, 1e-3)
    rows = int(min(w.M, max(16, rate * budget_s)))
    t0 = time.perf_counter()
    O.gemm(np.ascontiguousarray(A[:rows]), B, w.dtype, b_col=w.b_col)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / dt / 1e9, 2), "unit": "GFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"rows 0..{rows - 1} of C ({rows} x {w.N} outputs, full K={w.K}) of {w.name}; "
                      f"{dt:.1f} s on {cores} threads"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_from_profile(kernel_sha: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were
    taken on this exact kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_fp16_4096_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_sha:
        return None
    return d.get("hbm_bytes_per_launch")


def attention_bench():
    """The attention-style consumer (spt_attention) on its full-size workload under
    every producer: the pages' claim is that asynchronous copies stop paying once a
    tile load feeds many matrix instructions ("Kernel-Engpass analysieren", Schritt 4
    and the pitfalls: flash attention measured -5% with cp.async)."""
    import torch
    import software_pipelined_tiling_amd as spt
    from software_pipelined_tiling_amd import inputs as I
    w = I.W_ATTN_4096
    Q, K, V = (to_dev(x, w.dtype) for x in I.make_qkv(w))
    O = torch.empty((w.BH, w.Sq, w.D), dtype=torch.float32, device="cuda")
    scale = 1.0 / w.D ** 0.5
    res = {"workload": w.name + ", fp32 O, N(0,1) fp16 inputs, scale 1/sqrt(D)", "flop_per_call": w.flops,
           "alg_bytes_per_call": w.alg_bytes}
    for v, s_ in [("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2), ("direct", 3), ("auto", 0)]:
        def fn(stream, v=v, s_=s_):
            return spt.spt_attention(w.BH, w.Sq, w.Sk, w.D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                     scale, spt.DTYPE_CODES[w.dtype], stream, spt.VARIANT_CODES[v], s_) == 0
        us = time_graph(fn, calls=10, reps=5)
        if us is None:
            continue
        tf = w.flops / (us * 1e-6) / 1e12
        res[f"{v}{s_}"] = {"us": round(us, 2), "tflops": round(tf, 1),
                           "pct_of_peak": round(100 * tf / PEAK_TFLOPS[w.dtype], 1)}
    if "direct2" in res and "reg2" in res:
        best_d = min(res["direct2"]["us"], res["direct3"]["us"])
        best_r = min(res["reg1"]["us"], res["reg2"]["us"])
        res["async_over_register_staged"] = {
            "value": round(best_r / best_d, 3),
            "what": "time of the best register-staged ring / time of the best direct-to-LDS ring (> 1: the "
                    "asynchronous copies are faster); the pages measured 0.95 for flash attention on GA104",
            "pipelined_over_sync": round(res["sync1"]["us"] / min(best_d, best_r), 3)}
    # the compute/load ratio per key block (spt_attention.hip: 256 query rows, 32 keys of
    # 128 columns per block, 8 waves): 34 MFMAs per wave (32 of the two products, 2 row
    # sums) per 2 copies per thread
    res["ratio"] = {"mfma_per_copy": 17.0, "flop_per_byte": 256.0,
                    "gemm_headline_tile": {"mfma_per_copy": 8.0, "flop_per_byte": 128.0}}
    return res


def stream_bench(steps: int, warmup: int):
    """y = 2x ("Hiding Memory Latency ...", section 8) through spt_scale_by_two:
    8 bytes per element (one read, one write), HBM-bound."""
    import torch
    import software_pipelined_tiling_amd as spt
    out = {}
    stream = torch.cuda.current_stream()
    for name, n, blocks in (("pages demo: 2^20 floats, 1 block", 1 << 20, 1),
                            ("2^28 floats, 256 blocks (one per CU)", 1 << 28, 256),
                            ("2^28 floats, library blocks", 1 << 28, 0)):
        x = (torch.arange(n, device="cuda", dtype=torch.int64) % 113).to(torch.float32) * 0.25
        y = torch.empty_like(x)
        res = {}
        for s in (1, 2, 3, 4):
            def call():
                return spt.spt_scale_by_two(n, x.data_ptr(), y.data_ptr(), s, blocks, stream.cuda_stream)
            if call() != 0:
                raise RuntimeError(spt.spt_last_error())
            for _ in range(warmup):
                call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                call()
            e1.record(stream)
            e1.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            res[f"S{s}"] = {"us": round(us, 2), "gbs": round(8 * n / us / 1e3, 1),
                            "pct_of_hbm": round(100 * 8 * n / us / 1e3 / HBM_GBS, 1)}
        res["speedup_S3_vs_S1"] = round(res["S1"]["us"] / res["S3"]["us"], 3)
        if n == 1 << 28 and blocks == 0:  # context: torch's own elementwise multiply
            t = torch.empty_like(x)
            for _ in range(warmup):
                torch.mul(x, 2.0, out=t)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                torch.mul(x, 2.0, out=t)
            e1.record(stream)
            e1.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            res["torch_mul_reference"] = {"us": round(us, 2), "gbs": round(8 * n / us / 1e3, 1)}
            del t
        out[name] = res
        del x, y
    return out


_probe = None


def probe_lib():
    """libspt_probe.so (bench_probe.hip): the sustained-MFMA probe, a measurement
    tool kept out of libspt.so."""
    global _probe
    if _probe is None:
        import ctypes
        from software_pipelined_tiling_amd import build as B
        if not os.path.exists(B.PROBE_LIB):
            raise RuntimeError(f"{B.PROBE_LIB} not built (software_pipelined_tiling_amd.build.build_probe)")
        L = ctypes.CDLL(B.PROBE_LIB)
        L.spt_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.spt_probe_mfma.restype = ctypes.c_int
        _probe = L
    return _probe


def mfma_ceiling(prob: "Problem", seconds: float):
    """Sustained rate of MFMAs alone (spt_probe_mfma, no memory traffic in the
    loop) with the headline's own A matrix as operand data: the compute roof
    the power limit leaves for this data (context for the roofline fraction)."""
    import torch
    import software_pipelined_tiling_amd as spt
    stream = torch.cuda.current_stream()
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    nbytes = prob.dA.numel() * prob.dA.element_size()
    iters = 2000  # ~1 ms per launch
    code = spt.DTYPE_CODES[prob.w.dtype]

    def launch():
        return probe_lib().spt_probe_mfma(code, prob.dA.data_ptr(), nbytes, iters, sink.data_ptr(),
                                          stream.cuda_stream)
    if launch() != 0:
        return None
    for _ in range(100):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    t0 = time.perf_counter()
    e0.record(stream)
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            launch()
        torch.cuda.synchronize()
        n += 50
    e1.record(stream)
    e1.synchronize()
    ops = 256 * 4 * 64 * iters * (32768 if prob.w.dtype == "i8" else 16384) * n
    return round(ops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)


def mfma_ceilings(prob: "Problem", seconds: float):
    """mfma_ceiling with the headline's data, and with all-zero operands (the
    same instructions with no operand bits switching)."""
    import torch
    rate = mfma_ceiling(prob, seconds)
    keep = prob.dA
    prob.dA = torch.zeros_like(keep)
    try:
        rate0 = mfma_ceiling(prob, seconds)
    finally:
        prob.dA = keep
    return rate, rate0


def sample_power(prob: "Problem", seconds: float):
    """Run the headline call back to back for `seconds` while amd-smi samples
    socket power and the GFX (XCD) clocks; None when amd-smi is unavailable."""
    import re
    import shutil
    import subprocess
    import threading
    import torch
    import software_pipelined_tiling_amd as spt
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    samples, stop = [], [False]

    def poll():
        while not stop[0]:
            try:
                txt = subprocess.run([exe, "metric", "-p", "-c"], capture_output=True, text=True,
                                     timeout=20).stdout
            except Exception:
                return
            pw = re.findall(r"SOCKET_POWER:\s*(\d+)", txt)
            cl = [int(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)", txt)]
            if pw and cl:
                samples.append((int(pw[0]), sum(cl) / len(cl)))
            time.sleep(0.1)

    a = prob.args(torch.cuda.current_stream().cuda_stream)
    for _ in range(300):
        spt.spt_gemm_ex(*a)
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(100):
            spt.spt_gemm_ex(*a)
        torch.cuda.synchronize()
        n += 100
    dt = time.perf_counter() - t0
    stop[0] = True
    th.join(timeout=30)
    if len(samples) < 3:
        return None
    busy = samples[len(samples) // 3:]  # past the ramp
    watts = sorted(s[0] for s in busy)[len(busy) // 2]
    mhz = sorted(s[1] for s in busy)[len(busy) // 2]
    w = prob.w
    return {"socket_power_w": watts, "gfx_clock_mhz": round(mhz), "samples": len(busy),
            "sustained_tflops": round(w.flops * n / dt / 1e12, 1), "seconds": round(dt, 2),
            "peak_tflops_at_clock": round(FLOP_PER_CLK[w.dtype] * mhz * 1e6 / 1e12, 1),
            "source": "amd-smi metric -p -c, median after the first third of the samples"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed calls first; the GPU's clock settles within ~30 ms of load")
    ap.add_argument("--preheat", type=float, default=1.0,
                    help="seconds of untimed back-to-back headline calls before the warm-up (a fresh GPU "
                         "leaves its idle clocks over tens of ms; disclosed in the output)")
    ap.add_argument("--tile", type=int, default=0, help="headline tile (0 = library default)")
    ap.add_argument("--variant", default="auto", help="headline variant (auto/sync/reg/direct/persist)")
    ap.add_argument("--stages", type=int, default=0, help="headline stages (0 = variant default)")
    ap.add_argument("--cpu-budget", type=float, default=25.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-power", action="store_true", help="skip the amd-smi power / clock sample")
    ap.add_argument("--power-seconds", type=float, default=3.0)
    ap.add_argument("--only-headline", action="store_true", help="headline workload only (profiling)")
    ap.add_argument("--only-workload", default=None,
                    help="time only this side workload by name prefix, e.g. 'bf16 GEMM 8192' (profiling)")
    ap.add_argument("--only-attention", action="store_true",
                    help="besides the headline, time only the attention leg (profiling)")
    ap.add_argument("--auto-only", action="store_true",
                    help="side workloads: time only the library's default call (no unpipelined, vendor, "
                         "store-only or ceiling legs), so that a counter pass sees one kernel per workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 256 MiB device copies (HBM counter scale)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark runs on exactly one GPU; --gpus must be 1 "
              "(the GEMM shards over output tiles, see the sharding design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import software_pipelined_tiling_amd as spt
    from software_pipelined_tiling_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    spt.lib()  # fails loudly if libspt.so is missing

    head = Problem(I.W_F16_4096)
    w = head.w
    hv, hs, ht = args.variant, args.stages, args.tile
    if time_calls(head, 1, 0, hv, hs, ht) is None:
        print(f"bench.py: headline configuration refused: {spt.spt_last_error()}", file=sys.stderr)
        sys.exit(1)
    # untimed pre-heat (disclosed in the line), then W warm-up calls, then the timed region:
    # K back-to-back steps with a HIP event before the first and after every call
    t_pre = time.perf_counter()
    pre_calls = preheat(head, args.preheat, hv, hs, ht)
    t_pre = time.perf_counter() - t_pre
    ms = time_calls(head, args.steps, args.warmup, hv, hs, ht)
    # a second pass of K calls with an event after every call: the per-call spread (the
    # event records add a gap of a few us between kernels, so this pass runs slower)
    ms_each, per_call = time_calls_each(head, args.steps, 0, hv, hs, ht)
    tflops = w.flops / (ms * 1e-3) / 1e12
    rc, plan = spt.spt_plan(spt.F16, w.M, w.N, w.K, spt.ROW, spt.VARIANT_CODES[args.variant],
                            args.stages, args.tile)
    sha = kernel_source_hash()
    traffic = traffic_from_profile(sha)
    out = {
        "metric": "GEMM TFLOPS/TOPS at 4096^3 fp16 & int8, % of MI355X dense MFMA peak",
        "value": round(tflops, 1),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "timed_region": {"before": f"{pre_calls} untimed calls of the headline kernel back to back "
                                   f"({t_pre:.2f} s pre-heat), then {args.warmup} warm-up calls",
                         "events": "one HIP event before the first and one after the last timed call, "
                                   "on the launch stream, synchronised on both sides",
                         "per_call_pass": {
                             "what": f"{args.steps} more calls right after the timed region with an event after "
                                     "every call (the records add a gap between kernels)",
                             "ms_per_call": round(ms_each, 5),
                             "per_call_us": [round(x, 2) for x in per_call] if len(per_call) <= 100 else None,
                             "per_call_us_min_median_max": [round(min(per_call), 2),
                                                            round(sorted(per_call)[len(per_call) // 2], 2),
                                                            round(max(per_call), 2)]}},
        "config": {"workload": w.name + ", A/B row-major, fp32 accumulate, fp32 C, U[-1,1] fp16",
                   "tile": f"{plan.BM}x{plan.BN}x{plan.BK}", "threads": plan.threads,
                   "variant": {1: "sync", 2: "reg", 3: "direct", 4: "persist"}[plan.variant],
                   "stages": plan.stages, "pct_of_peak": round(100 * tflops / PEAK_TFLOPS["f16"], 1)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_TFLOPS["f16"],
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS["f16"], 4),
                     "traffic": traffic, "kernel_source_sha": sha,
                     "alg_flop_per_launch": w.flops, "alg_bytes_per_launch": w.alg_bytes},
    }

    if args.copy_calibration:
        # a plain copy of known size: 256 MiB read + 256 MiB written per launch
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel() * 4
        del src, dst

    if not args.only_headline and not args.no_power:
        out["power"] = sample_power(head, args.power_seconds)
        ceil, ceil0 = mfma_ceilings(head, 2.0)
        if ceil:
            out["mfma_ceiling"] = {"tflops": ceil, "value_over_ceiling": round(tflops / ceil, 4),
                                   "zero_operands_tflops": ceil0,
                                   "what": "spt_probe_mfma: 16x16x32 fp16 MFMAs alone, operands = the headline's "
                                           "A matrix (and, for comparison, zeros), one wave per SIMD on every CU, "
                                           "sustained 2 s each"}

    if not args.only_headline:
        vu = vendor_us(head)
        if vu:
            out["vendor_hipblaslt"] = {"us": vu, "tflops": round(w.flops / (vu * 1e-6) / 1e12, 1),
                                       "value_over_vendor": round(vu / (ms * 1e3), 3),
                                       "what": "torch.mm(A, B, out_dtype=float32) on the same operands (context)"}

    if args.only_workload or args.only_attention:
        args.no_sweep = True
    if not args.only_headline:
        steps = max(20, min(args.steps, 100))
        if not args.no_sweep:
            sweep = []
            for tile in TILES:
                for v, s in PAIRS:
                    t = time_calls(head, steps, 20, v, s, tile)
                    if t is None:
                        continue
                    sweep.append({"tile": tile, "variant": v, "stages": s, "us": round(t * 1e3, 2),
                                  "tflops": round(w.flops / (t * 1e-3) / 1e12, 1)})
            out["sweep"] = sweep
            by = {(d["tile"], d["variant"], d["stages"]): d["tflops"] for d in sweep}
            # speedup of each pipelined form over the unpipelined SYNC loop of the same tile:
            # the pages' 128 x 256 x 32 tile, and the tile of the headline
            pg = by.get((1, "direct", 3))
            if pg:  # the pages' shape: 128 x 256 x 32 fp16 tile, 256 threads, 3-stage ring
                out["pages_shape"] = {"tile": "128x256x32", "threads": 256, "variant": "direct", "stages": 3,
                                      "tflops": pg, "pct_of_peak": round(100 * pg / PEAK_TFLOPS["f16"], 1),
                                      "speedup_vs_unpipelined": round(pg / by[(1, "sync", 1)], 3)
                                      if (1, "sync", 1) in by else None}
            for name, t in (("pipelining_speedup_pages_tile", 1), ("pipelining_speedup_headline_tile", plan.tile_id)):
                base = by.get((t, "sync", 1))
                if base:
                    out[name] = {f"{v}{s}": round(by[(t, v, s)] / base, 3) for v, s in PAIRS if (t, v, s) in by}
        del head
        extra = {}
        for wk in [I.W_I8_4096, I.W_BF16_RAGGED, I.W_F16_256] + [I.w_bf16_lowk(k) for k in I.LOWK_KS]:
            if (args.only_workload and not wk.name.startswith(args.only_workload)) or args.only_attention:
                continue
            p = Problem(wk)
            us = gemm_us(p)
            peak = PEAK_TFLOPS[wk.dtype]
            tf = wk.flops / (us * 1e-6) / 1e12
            gbs = wk.alg_bytes / (us * 1e-6) / 1e9
            extra[wk.name] = {"us": us, "tflops": round(tf, 1), "pct_of_peak": round(100 * tf / peak, 1),
                              "hbm_gbs_alg": round(gbs, 1), "pct_of_hbm": round(100 * gbs / HBM_GBS, 1)}
            if args.auto_only:  # (counter passes: the library's own call only)
                del p
                continue
            us1 = gemm_us(p, "sync", 1)
            extra[wk.name].update({"unpipelined_us": us1, "speedup_vs_unpipelined": round(us1 / us, 3)})
            extra[wk.name]["vendor_hipblaslt_us"] = vendor_us(p)
            if wk is I.W_F16_256:
                # the small case: the single-stage loop beside the 2-stage (and deeper) pipelines,
                # on the tile the library picks and on the pages' 128 x 256 x 32 tile
                rc, pp = spt.spt_plan(spt.F16, wk.M, wk.N, wk.K, spt.ROW)
                for tile in sorted({pp.tile_id, 1}):
                    row = {}
                    for v, s_ in PAIRS:
                        tv = gemm_us(p, v, s_, tile)
                        if tv is not None:
                            row[f"{v}{s_}"] = tv
                    extra[wk.name][f"variants_us_tile{tile}"] = row
            if wk.K <= 1024 and wk.M * wk.N >= 1 << 24:
                # the C store alone: the same kernel with K = 0 (it writes zeros to all of C)
                extra[wk.name]["c_store_only_us"] = c_store_only(p)
            if wk is I.W_I8_4096 and not args.no_power:  # the int8 compute roof for this data
                ceil = mfma_ceiling(p, 2.0)
                if ceil:
                    extra[wk.name]["mfma_ceiling_tops"] = ceil
                    extra[wk.name]["value_over_ceiling"] = round(tf / ceil, 4)
            del p
        out["workloads"] = extra
        out["workloads_timing"] = ("every side workload: 20 calls captured in one HIP graph, replayed untimed for "
                                   "20 ms, then 10 times with an event pair around each replay; the median replay "
                                   "over 20 (GPU time of back-to-back calls)")

        if not args.only_workload and not args.only_attention:
            out["streaming"] = stream_bench(steps, 20)
        if not args.only_workload:
            out["attention"] = attention_bench()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(I.W_F16_4096, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
