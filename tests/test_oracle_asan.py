"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

`tests/oracle_asan_driver.c` calls every entry point of `oracle/oracle.c` with
operand buffers cut to exactly the bytes the layout contract reads, over
padded pitches, both B layouts, K = 0, empty outputs, the int8 K limit and
the refused arguments.  Built with gcc and run here; any out-of-bounds
access, use after free, leak or signed overflow fails the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_is_clean_under_the_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    exe = str(tmp_path / "oracle_asan")
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(HERE, "oracle_asan_driver.c"), "-lm"],
        capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("gcc without sanitizer runtimes: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "oracle ok under the sanitizers" in run.stdout
