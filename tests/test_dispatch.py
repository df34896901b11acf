"""The dispatcher launches the grid its plan reports (CPU only).

`tests/dispatch_driver.cpp` links the library's host code with kernel tables
whose launchers only record the grid and kernel arguments, so the launches
of `spt_gemm_ex` can be compared with `spt_plan` without a GPU:
- the persistent variant launches at most the 512 resident workgroups, each
  walking a stream of output tiles (the grid `spt_plan` reports), never one
  workgroup per tile;
- the one-tile variants launch one workgroup per output tile;
- AUTO's row band is two launches: the whole rows of tiles before the band,
  then the band's 128 x 128 tiles, with the grids and rows the plan gives.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
F16, BF16, I8, F32 = 0, 1, 2, 3
AUTO, SYNC, REG, DIRECT, PERSIST = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers not installed")
    exe = str(tmp_path_factory.mktemp("dispatch") / "dispatch")
    r = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-o", exe,
         os.path.join(ROOT, "software_pipelined_tiling_amd", "csrc", "spt_api.cpp"),
         os.path.join(HERE, "dispatch_driver.cpp"), "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(ROCM, "lib")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    def run(cases):
        inp = "".join(" ".join(str(x) for x in c) + "\n" for c in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, timeout=60)
        assert out.returncode == 0, out.stderr
        res, cur = [], None
        for line in out.stdout.splitlines():
            f = line.split()
            if f[0] == "plan":
                cur = {"plan_rc": int(f[1]), "grid": int(f[2]), "tiles_m": int(f[3]), "tiles_n": int(f[4]),
                       "band_grid": int(f[5]), "band_m": int(f[6]), "variant": int(f[7]), "tile": int(f[8]),
                       "launches": []}
            elif f[0] == "launch":
                cur["launches"].append(dict(zip(("grid", "M", "tiles_m", "tiles_n", "k_full", "k_tail"),
                                                map(int, f[1:]))))
            else:
                cur["rc"] = int(f[1])
                res.append(cur)
        assert len(res) == len(cases)
        return res
    return run


PERSIST_SHAPES = [(BF16, 0, 8192, 8192, 512), (BF16, 0, 8192, 8192, 64), (F16, 0, 4096, 4096, 256),
                  (I8, 1, 4096, 4096, 512), (F32, 0, 2048, 2048, 64), (F16, 1, 1024, 1024, 256),
                  (BF16, 0, 128, 128, 128)]


@pytest.mark.parametrize("dt,lay,M,N,K", PERSIST_SHAPES)
@pytest.mark.parametrize("stages", [2, 3, 4])
def test_persistent_grid_is_the_resident_workgroups(driver, dt, lay, M, N, K, stages):
    (r,) = driver([(dt, lay, PERSIST, stages, 0, M, N, K)])
    k_tiles = K // (64 // {F16: 2, BF16: 2, I8: 1, F32: 4}[dt])
    if stages == 4 and k_tiles < 4:
        assert r["rc"] == -2  # a 4-stage persistent ring needs at least 4 K tiles
        return
    assert r["plan_rc"] == 0 and r["rc"] == 0
    tiles = r["tiles_m"] * r["tiles_n"]
    assert r["grid"] == min(tiles, 512)
    assert len(r["launches"]) == 1
    (l,) = r["launches"]
    assert l["grid"] == r["grid"] <= 512
    assert (l["tiles_m"], l["tiles_n"]) == (r["tiles_m"], r["tiles_n"])


@pytest.mark.parametrize("variant,stages,tile", [(SYNC, 1, 1), (REG, 2, 1), (DIRECT, 3, 1), (DIRECT, 2, 4),
                                                 (DIRECT, 4, 3), (DIRECT, 3, 4), (DIRECT, 3, 2), (AUTO, 0, 0)])
@pytest.mark.parametrize("dt,lay,M,N,K", [(F16, 0, 4096, 4096, 4096), (BF16, 0, 4000, 3000, 1000),
                                          (I8, 1, 8192, 8192, 512), (F32, 0, 300, 600, 333),
                                          (F16, 0, 4096, 4096, 0)])
def test_one_tile_variants_launch_one_workgroup_per_tile(driver, variant, stages, tile, dt, lay, M, N, K):
    (r,) = driver([(dt, lay, variant, stages, tile, M, N, K)])
    assert r["plan_rc"] == 0 and r["rc"] == 0, r
    if r["band_grid"]:
        pytest.skip("AUTO chose a row band here (covered below)")
    assert len(r["launches"]) == 1
    (l,) = r["launches"]
    assert l["grid"] == r["grid"] == r["tiles_m"] * r["tiles_n"]
    assert l["M"] == M


@pytest.mark.parametrize("dt,lay,M,N,K", [(F16, 0, 4352, 4096, 8192), (I8, 1, 4100, 4112, 4112),
                                          (BF16, 0, 6000, 6000, 2000), (F32, 0, 4100, 4100, 1024),
                                          (F16, 0, 4608, 5120, 4096)])
def test_row_band_launches_main_rows_then_band(driver, dt, lay, M, N, K):
    (r,) = driver([(dt, lay, AUTO, 0, 0, M, N, K)])
    assert r["rc"] == 0 and r["band_grid"] > 0, r
    main, band = r["launches"]
    assert main["grid"] == r["grid"] == main["tiles_m"] * main["tiles_n"]
    assert main["M"] == r["band_m"] and main["tiles_n"] == r["tiles_n"]
    assert band["grid"] == r["band_grid"] == band["tiles_m"] * band["tiles_n"]
    assert band["M"] == M - r["band_m"] and band["tiles_m"] * 128 >= band["M"] > (band["tiles_m"] - 1) * 128
