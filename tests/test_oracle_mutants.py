"""Planted mistakes in the oracle must each break at least one pin (CPU only).

Each mutant wraps the oracle with one plausible implementation mistake -- a
dropped k term, a transposed operand, a wrong sign, an index shifted by one,
a swapped loop bound -- and must fail at least one of the pins that the real
oracle passes.  This shows the pins can see such mistakes.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests import oracle_pins


def _logical_b(B, b_col, K, N):
    """The logical K x N matrix of stored B as an array (row-major copy)."""
    return np.ascontiguousarray(B[:N, :K].T) if b_col else np.ascontiguousarray(B[:K, :N])


def mut_drop_last_k(A, B, dtype, b_col=False, K=None, N=None):
    K = A.shape[1] if K is None else K
    if K == 0:
        return O.gemm(A, B, dtype, b_col=b_col, K=K, N=N)
    return O.gemm(A, B, dtype, b_col=b_col, K=K - 1, N=N)


def mut_drop_first_k(A, B, dtype, b_col=False, K=None, N=None):
    K = A.shape[1] if K is None else K
    N = (B.shape[0] if b_col else B.shape[1]) if N is None else N
    if K <= 1:
        return O.gemm(A, B, dtype, b_col=b_col, K=K, N=N)
    Bl = _logical_b(B, b_col, K, N)
    return O.gemm(np.ascontiguousarray(A[:, 1:K]), np.ascontiguousarray(Bl[1:]), dtype)


def mut_transpose_b(A, B, dtype, b_col=False, K=None, N=None):
    # read B with the other layout flag (a transposed operand)
    K = A.shape[1] if K is None else K
    N = (B.shape[0] if b_col else B.shape[1]) if N is None else N
    Bl = _logical_b(B, b_col, K, N)
    if Bl.shape[0] != Bl.shape[1]:
        return O.gemm(A, B, dtype, b_col=b_col, K=K, N=N) * 1.0 + 1.0  # shape mismatch: wrong anyway
    return O.gemm(A, np.ascontiguousarray(Bl.T), dtype, K=K)


def mut_negate_last_term(A, B, dtype, b_col=False, K=None, N=None):
    K = A.shape[1] if K is None else K
    C = O.gemm(A, B, dtype, b_col=b_col, K=K, N=N).astype(np.float64)
    if K == 0:
        return C
    last = O.gemm(np.ascontiguousarray(A[:, K - 1:K]),
                  np.ascontiguousarray(_logical_b(B, b_col, K, C.shape[1])[K - 1:K]), dtype)
    return C - 2.0 * last


def mut_shift_a_index(A, B, dtype, b_col=False, K=None, N=None):
    # A[i][k+1] used in place of A[i][k] (wraps at the end)
    K = A.shape[1] if K is None else K
    As = np.ascontiguousarray(np.roll(A[:, :K], -1, axis=1))
    return O.gemm(As, B, dtype, b_col=b_col, K=K, N=N)


def mut_shift_output_row(A, B, dtype, b_col=False, K=None, N=None):
    C = O.gemm(A, B, dtype, b_col=b_col, K=K, N=N)
    return np.roll(C, 1, axis=0)


def mut_m_loop_short(A, B, dtype, b_col=False, K=None, N=None):
    C = O.gemm(A, B, dtype, b_col=b_col, K=K, N=N).astype(np.float64)
    if C.shape[0]:
        C[-1, :] = 0.0  # the last output row never written
    return C


def mut_sum_truncated_to_input_precision(A, B, dtype, b_col=False, K=None, N=None):
    # accumulating in the input format instead of a wide accumulator
    C = O.gemm(A, B, dtype, b_col=b_col, K=K, N=N).astype(np.float64)
    if dtype == "f16":
        return C.astype(np.float16).astype(np.float64)
    if dtype == "i8":
        return ((C.astype(np.int64) + 128) % 256 - 128).astype(np.float64)
    return C.astype(np.float32).astype(np.float64) * (1 + 2.0 ** -20)


MUTANTS = [mut_drop_last_k, mut_drop_first_k, mut_transpose_b, mut_negate_last_term,
           mut_shift_a_index, mut_shift_output_row, mut_m_loop_short,
           mut_sum_truncated_to_input_precision]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "i8"])
@pytest.mark.parametrize("b_col", [False, True])
def test_mutant_is_caught(oracle_mod, mutant, dtype, b_col):
    res = oracle_pins.run_all(mutant, dtype, b_col)
    assert not all(res.values()), f"{mutant.__name__} passed every pin: {res}"
