"""The CPU oracle against facts fixed outside it (no GPU).

The oracle writes out C[i][j] = sum_k A[i][k] B[k][j] ("Pipeline GPU Kernel",
Schritt 5: pipelining leaves the arithmetic unchanged).  These tests pin it
with the identity, a permutation, rank-1 closed forms, exact integer
products (numpy int64 matmul), brute force on every tiny shape, numpy's
float64 matmul, padding, the empty sum and both layouts of B.
"""
import numpy as np
import pytest

from software_pipelined_tiling_amd.inputs import draw
from tests import oracle_pins

DTYPES = ["f16", "bf16", "f32", "i8"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("b_col", [False, True])
def test_pins_hold(oracle_mod, dtype, b_col):
    res = oracle_pins.run_all(oracle_mod.gemm, dtype, b_col)
    assert all(res.values()), res


def test_f16_decode_all_patterns(oracle_mod):
    """Every one of the 65536 binary16 patterns decodes to numpy's own float16 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_decode_known_values(oracle_mod):
    """bfloat16 patterns with textbook values (sign, 8-bit exponent bias 127, 7-bit fraction)."""
    cases = {
        0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC000: -2.0, 0x4049: 3.140625,
        0x3F00: 0.5, 0x3E80: 0.25, 0x4120: 10.0, 0x42C8: 100.0, 0x7F7F: 3.3895313892515355e38,
        0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x7F80: np.inf, 0xFF80: -np.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle_mod.decode(bits, "bf16")
    assert got.tolist() == list(cases.values())
    assert np.isnan(oracle_mod.decode(np.array([0x7FC0], dtype=np.uint16), "bf16")[0])


def test_f16_decode_known_values(oracle_mod):
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24,
             0x3555: 0.333251953125, 0x7C00: np.inf, 0x8000: -0.0}
    got = oracle_mod.decode(np.array(list(cases), dtype=np.uint16), "f16")
    assert got.tolist() == list(cases.values())


def test_empty_m_or_n(oracle_mod):
    A = np.zeros((0, 8), dtype=np.uint16)
    B = np.zeros((8, 5), dtype=np.uint16)
    assert oracle_mod.gemm(A, B, "f16").shape == (0, 5)
    A = np.zeros((3, 8), dtype=np.int8)
    B = np.zeros((8, 0), dtype=np.int8)
    assert oracle_mod.gemm(A, B, "i8").shape == (3, 0)


def test_int8_extremes_and_k_bound(oracle_mod):
    """(-128)*(-128) summed 4096 times is 2^26 exactly; K beyond the exact-int32 bound is refused."""
    A = np.full((3, 4096), -128, dtype=np.int8)
    B = np.full((4096, 2), -128, dtype=np.int8)
    C = oracle_mod.gemm(A, B, "i8")
    assert C.dtype == np.int32 and np.all(C == 4096 * 16384)
    A = np.full((1, 131071), -128, dtype=np.int8)
    B = np.full((1, 131071), -128, dtype=np.int8)  # column-major, N = 1
    assert oracle_mod.gemm(A, B, "i8", b_col=True)[0, 0] == 131071 * 16384
    with pytest.raises(ValueError):
        oracle_mod.gemm(np.zeros((1, 131072), np.int8), np.zeros((1, 131072), np.int8), "i8",
                        b_col=True)


@pytest.mark.parametrize("dtype", DTYPES)
def test_entries_match_full(oracle_mod, dtype):
    rng = np.random.default_rng(7)
    lo, hi = (-128, 127) if dtype == "i8" else (-1, 1)
    A = draw("uniform", lo, hi, (37, 70), rng, dtype)
    B = draw("uniform", lo, hi, (70, 29), rng, dtype)
    full = oracle_mod.gemm(A, B, dtype)
    r = rng.integers(0, 37, 200)
    c = rng.integers(0, 29, 200)
    ent = oracle_mod.gemm_entries(A, B, dtype, r, c)
    assert np.array_equal(ent, full[r, c])
    Bc = np.ascontiguousarray(B.T)
    assert np.array_equal(oracle_mod.gemm_entries(A, Bc, dtype, r, c, b_col=True), full[r, c])


def test_thread_count_invariant(oracle_mod):
    rng = np.random.default_rng(3)
    A = draw("uniform", -1, 1, (64, 96), rng, "bf16")
    B = draw("uniform", -1, 1, (96, 48), rng, "bf16")
    assert np.array_equal(oracle_mod.gemm(A, B, "bf16", threads=1),
                          oracle_mod.gemm(A, B, "bf16", threads=4))


def test_integer_valued_fp16_exact_at_size(oracle_mod):
    """Integer inputs in [-4, 4]: every partial sum is an integer below 2^24, so the
    result equals numpy's int64 matmul exactly."""
    rng = np.random.default_rng(11)
    A = draw("intgrid", -4, 4, (128, 512), rng, "f16")
    B = draw("intgrid", -4, 4, (512, 96), rng, "f16")
    Ai = A.view(np.float16).astype(np.int64)
    Bi = B.view(np.float16).astype(np.int64)
    assert np.array_equal(oracle_mod.gemm(A, B, "f16"), (Ai @ Bi).astype(np.float64))
