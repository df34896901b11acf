"""Build libspt.so (the gfx950 HIP kernels + the C ABI of include/spt.h).

Every translation unit is compiled by hipcc for gfx950 in parallel, then
linked into ``software_pipelined_tiling_amd/libspt.so`` (in-tree).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [f"spt_kernels_{dt}_{lay}.hip" for dt in ("f16", "bf16", "i8", "f32") for lay in ("row", "col")]
SOURCES += ["spt_stream.hip", "spt_attention.hip", "spt_api.cpp"]
HEADERS = ["spt_kernel.hpp", "spt_persist.hpp", "spt_instances.hpp", "spt_registry.h", "spt_config.h"]

# Packed-fp32 VALU instructions are disabled for all device code (-packed-fp32-ops).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-command-line-argument"]
# The attention kernel keeps its MFMA results in ordinary VGPRs, where its softmax
# works on them; the GEMM kernels' 256 accumulators per lane need the AGPRs.
SOURCE_FLAGS = {"spt_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def build_all(verbose: bool = True) -> None:
    """libspt.so, the race-detection libspt_poison.so and bench.py's measurement
    probe libspt_probe.so, compiled side by side."""
    with cf.ThreadPoolExecutor(max_workers=3) as ex:
        for f in [ex.submit(build, verbose=verbose), ex.submit(build_poison, verbose=verbose),
                  ex.submit(build_probe, verbose=verbose)]:
            f.result()


def build(jobs: int | None = None, verbose: bool = True, defines=(), out: str | None = None,
          reuse: bool = False, only=()) -> str:
    """Compile every source for gfx950 and link libspt.so (or `out`); returns its path.

    `defines` are extra preprocessor definitions (tuning experiments only).
    With `reuse`, sources not listed in `only` keep their existing object file."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    tag = "" if not defines else "_" + str(abs(hash(tuple(defines))))

    def obj(src):
        o = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
        if reuse and src not in only and os.path.exists(o):
            return o
        return _compile(src, defines, tag)

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(obj, SOURCES))
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", file=sys.stderr)
    return lib


POISON_LIB = os.path.join(HERE, "libspt_poison.so")
POISON_TABLES = ("f16_row", "i8_col")


def build_poison(verbose: bool = True) -> str:
    """The race-detection library ``libspt_poison.so``: the same C ABI, built with
    SPT_POISON, so that every ring refills a freed stage only after poisoning it.
    It holds the kernel tables of fp16 with row-major B and int8 with column-major B;
    the other element types and layouts have empty tables (SPT_ERR_UNSUPPORTED).
    Test infrastructure: the product loads libspt.so only."""
    os.makedirs(BUILD, exist_ok=True)
    stub = os.path.join(BUILD, "spt_poison_stub.cpp")
    empty = [f"{dt}_{lay}" for dt in ("f16", "bf16", "i8", "f32") for lay in ("row", "col")
             if f"{dt}_{lay}" not in POISON_TABLES]
    with open(stub, "w") as f:
        f.write('#include "spt_registry.h"\nnamespace spt {\n')
        f.writelines(f"KernelTable kernels_{t}() {{ return KernelTable{{nullptr, 0}}; }}\n" for t in empty)
        f.write("}\n")
    srcs = [f"spt_kernels_{t}.hip" for t in POISON_TABLES] + ["spt_stream.hip", "spt_attention.hip", "spt_api.cpp"]
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, ("SPT_POISON",), "_poison"), srcs))
    stub_obj = os.path.join(BUILD, "spt_poison_stub.o")
    r = subprocess.run([HIPCC, *COMMON, "-I", CSRC, "-c", stub, "-o", stub_obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the poison stub:\n{r.stderr[-4000:]}")
    tmp = POISON_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, stub_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, POISON_LIB)
    if verbose:
        print(f"built {POISON_LIB}", file=sys.stderr)
    return POISON_LIB


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(HERE, "libspt_probe.so")


def build_probe(verbose: bool = True) -> str:
    """``libspt_probe.so``: the sustained-MFMA probe that bench.py loads (a
    measurement tool, not part of libspt.so or its C ABI)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-I", ROOT, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the probe:\n{r.stderr[-4000:]}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}", file=sys.stderr)
    return PROBE_LIB


def asm(src: str = "spt_kernels_f16_row.hip", out: str | None = None) -> str:
    """gfx950 assembly of one kernel translation unit (for the ISA checks)."""
    os.makedirs(BUILD, exist_ok=True)
    out = out or os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-4000:]}")
    return out


if __name__ == "__main__":
    build_all()
