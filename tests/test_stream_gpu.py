"""Parity of the streaming pipeline y = 2x (through the C ABI) with the CPU
oracle, on an MI355X ("Hiding Memory Latency ...", sections 8 and 9).

Doubling is exact, so every result must equal the oracle bit for bit (NaN
inputs: NaN outputs).  y is over-allocated and pre-filled with a sentinel so
a write past n shows up.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import software_pipelined_tiling_amd as spt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SENT = np.uint32(0x7FC0DEAD)
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_stream_example.json")))


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


def random_input(n, seed):
    """Finite values over a wide exponent range, plus signed zeros, infinities,
    subnormals and NaN at fixed places."""
    rng = np.random.default_rng([11, n, seed])
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, 3.4e38, -1.7e38], np.float32)
    k = min(n, special.size)
    x[:k] = special[:k]
    return x


def run(x, stages, blocks, inplace=False, stream=None):
    n = x.size
    dx = torch.from_numpy(x.copy()).cuda()
    if inplace:
        dy = dx
    else:
        dy = torch.from_numpy(np.full(n + 64, SENT, np.uint32)).cuda().view(torch.float32)
    s = torch.cuda.current_stream() if stream is None else stream
    rc = spt.spt_scale_by_two(n, dx.data_ptr(), dy.data_ptr(), stages, blocks, s.cuda_stream)
    assert rc == 0, spt.spt_last_error()
    torch.cuda.synchronize()
    y = dy.cpu().numpy()
    if not inplace:
        assert np.all(y[n:].view(np.uint32) == SENT), "write past n"
    return y[:n]


def same(got, want):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_pages_example(oracle_mod):
    """The pages' demonstration: 2^20 elements (i mod 113) * 0.25, one block of
    256 threads, 3 stages: max_error = 0 as printed."""
    n = GOLDEN["n"]
    x = ((np.arange(n) % 113).astype(np.float32) * np.float32(0.25))
    y = run(x, GOLDEN["stages"], GOLDEN["blocks"])
    assert float(np.max(np.abs(y.astype(np.float64) - 2.0 * x.astype(np.float64)))) == GOLDEN["printed_max_error"]
    same(y, oracle_mod.scale_by_two(x))


@pytest.mark.parametrize("stages", [1, 2, 3, 4])
@pytest.mark.parametrize("blocks", [1, 3, 0])
def test_ragged_lengths(oracle_mod, stages, blocks):
    """Lengths around every boundary: inside one chunk, one tile, several tiles,
    and n not a multiple of 4 (the straddling chunk)."""
    for i, n in enumerate([1, 2, 3, 4, 5, 255, 1023, 1024, 1025, 2048, 4095, 3 * 1024 + 7, 10 * 1024 + 1,
                           (1 << 16) + 3]):
        x = random_input(n, i)
        same(run(x, stages, blocks), oracle_mod.scale_by_two(x))


@pytest.mark.parametrize("stages", [1, 3])
def test_in_place(oracle_mod, stages):
    x = random_input(50_001, 5)
    same(run(x, stages, 0, inplace=True), oracle_mod.scale_by_two(x))


def test_many_blocks_large(oracle_mod):
    """2^26 + 5 elements (256 MiB) with the library's block count."""
    x = random_input((1 << 26) + 5, 9)
    same(run(x, 0, 0), oracle_mod.scale_by_two(x))


def test_more_blocks_than_tiles_and_other_stream(oracle_mod):
    x = random_input(5000, 3)
    same(run(x, 2, 1000, stream=torch.cuda.Stream()), oracle_mod.scale_by_two(x))


def test_torch_wrapper(oracle_mod):
    x = random_input(12345, 4)
    y = spt.scale_by_two(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    same(y.cpu().numpy(), oracle_mod.scale_by_two(x))


def test_torch_wrapper_rejects_host_tensors():
    """A host tensor never reaches the kernel (its pointer is not a device address)."""
    with pytest.raises(ValueError):
        spt.scale_by_two(torch.ones(1024))
    with pytest.raises(ValueError):
        spt.scale_by_two(torch.ones(1024, device="cuda"), out=torch.empty(1024))
