"""bench.py's contract on the CPU side (no GPU needed): it refuses more than one
GPU with a message, exits cleanly without a GPU, and reports HBM traffic only
from counter summaries taken on the kernel sources it runs."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run(env=env)
    assert r.returncode == 2


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and os.path.exists("/dev/kfd"),
                    reason="a GPU may be visible here")
def test_no_gpu_exits_with_a_message():
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "no GPU" in r.stderr


def test_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    assert len(sha) == 16 and sha == bench.kernel_source_hash()  # deterministic
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemm_fp16_4096_hbm_traffic.json").write_text(
        json.dumps({"kernel_source_sha": sha, "hbm_bytes_per_launch": 12345}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile(sha) == 12345
    assert bench.traffic_from_profile("0" * 16) is None
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "nowhere"))
    assert bench.traffic_from_profile(sha) is None
