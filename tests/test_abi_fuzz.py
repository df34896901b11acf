"""The C ABI's argument checks fuzzed under AddressSanitizer and UBSan (CPU only).

`tests/abi_fuzz_driver.cpp` links the library's host code
(`software_pipelined_tiling_amd/csrc/spt_api.cpp`) with empty kernel tables
and failing launchers, so no call can reach a GPU, and drives every entry
point with 400000 argument sets over edge values: sizes and pitches around
tile, 2^31 and 2^63 limits, null, misaligned, overlapping and out-of-range
pointers, every enum value and values past each end.  Each call must return
one of the five status codes, OK only where nothing is to be launched, with
a message exactly when it failed; any memory error or undefined behaviour in
the checks fails the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_checks_under_the_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers not installed")
    exe = str(tmp_path / "abi_fuzz")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
         os.path.join(ROOT, "software_pipelined_tiling_amd", "csrc", "spt_api.cpp"),
         os.path.join(HERE, "abi_fuzz_driver.cpp"), "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(ROCM, "lib")],
        capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("g++ without sanitizer runtimes: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-4000:])
    assert "abi checks ok under the sanitizers: 400000 rounds" in run.stdout
    # the generator reaches the late checks too, not only the early refusals (the
    # driver's tally prints each message with its digits removed)
    for msg in ("C overlaps A or B", "too many output tiles", "C or ldc not -byte aligned",
                "outside the device address range", "no kernel built", "exceeds the  KiB"):
        assert msg in run.stdout, msg
