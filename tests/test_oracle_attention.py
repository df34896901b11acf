"""The attention oracle against its pins, planted mistakes, and its argument
checks (CPU only)."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from software_pipelined_tiling_amd.inputs import draw
from tests import attention_pins as P


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pin", P.PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(oracle_mod, dtype, pin):
    assert pin(O.attention, dtype, np.random.default_rng(7))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_oracle_matches_numpy_float64(oracle_mod, dtype):
    """Random inputs: numpy's float64 matmul, max, exp and sum as library steps."""
    rng = np.random.default_rng(3)
    Q = draw("uniform", -1, 1, (3, 37, 64), rng, dtype)
    K = draw("uniform", -1, 1, (3, 53, 64), rng, dtype)
    V = draw("normal", 0, 1, (3, 53, 64), rng, dtype)
    q, k, v = (P._values(x, dtype) for x in (Q, K, V))
    s = 0.125 * q @ k.transpose(0, 2, 1)
    e = np.exp(s - s.max(axis=2, keepdims=True))
    want = (e / e.sum(axis=2, keepdims=True)) @ v
    assert np.max(np.abs(O.attention(Q, K, V, dtype, 0.125) - want)) < 1e-12


def test_rows_entry_point_equals_full(oracle_mod):
    rng = np.random.default_rng(4)
    Q = draw("uniform", -1, 1, (2, 19, 16), rng, "f16")
    K = draw("uniform", -1, 1, (2, 23, 16), rng, "f16")
    V = draw("uniform", -1, 1, (2, 23, 16), rng, "f16")
    full = O.attention(Q, K, V, "f16", 0.25)
    sl, rw = np.array([0, 1, 1, 0]), np.array([0, 18, 5, 7])
    assert np.array_equal(O.attention_rows(Q, K, V, "f16", 0.25, sl, rw), full[sl, rw])


def test_argument_checks(oracle_mod):
    Q = np.zeros((1, 2, 4), np.uint16)
    K = np.zeros((1, 0, 4), np.uint16)
    with pytest.raises(ValueError):  # a softmax over no keys is undefined
        O.attention(Q, K, K, "f16", 1.0)
    with pytest.raises(ValueError):
        O.attention_rows(Q, np.zeros((1, 3, 4), np.uint16), np.zeros((1, 3, 4), np.uint16), "f16", 1.0, [1], [0])
    assert O.attention(np.zeros((0, 2, 4), np.uint16), np.zeros((0, 3, 4), np.uint16),
                       np.zeros((0, 3, 4), np.uint16), "f16", 1.0).shape == (0, 2, 4)


# ---- planted mistakes: each must break at least one pin --------------------------------
def _v(x, dtype):
    return P._values(np.asarray(x), dtype)


def _ref(q, k, v, scale, *, sub_max=True, norm=True, axis=2):
    s = scale * q @ k.transpose(0, 2, 1)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s - s.max(axis=axis, keepdims=True)) if sub_max else np.exp(s)
        p = e / e.sum(axis=axis, keepdims=True) if norm else e
        return p @ v


def mut_no_max_subtraction(Q, K, V, dtype, scale):
    return _ref(_v(Q, dtype), _v(K, dtype), _v(V, dtype), scale, sub_max=False)


def mut_no_normalisation(Q, K, V, dtype, scale):
    return _ref(_v(Q, dtype), _v(K, dtype), _v(V, dtype), scale, norm=False)


def mut_softmax_over_queries(Q, K, V, dtype, scale):
    return _ref(_v(Q, dtype), _v(K, dtype), _v(V, dtype), scale, axis=1)


def mut_scale_ignored(Q, K, V, dtype, scale):
    return O.attention(Q, K, V, dtype, 1.0)


def mut_scale_squared(Q, K, V, dtype, scale):
    return O.attention(Q, K, V, dtype, scale * scale)


def mut_keys_as_values(Q, K, V, dtype, scale):
    return O.attention(Q, K, K, dtype, scale)


def mut_values_shifted(Q, K, V, dtype, scale):
    return O.attention(Q, K, np.ascontiguousarray(np.roll(V, 1, axis=1)), dtype, scale)


def mut_last_key_dropped(Q, K, V, dtype, scale):
    if K.shape[1] < 2:
        return O.attention(Q, K, V, dtype, scale)
    return O.attention(Q, np.ascontiguousarray(K[:, :-1]), np.ascontiguousarray(V[:, :-1]), dtype, scale)


def mut_head_dim_transposed(Q, K, V, dtype, scale):
    # keys read with their last two axes swapped where square (a transposed operand)
    if K.shape[1] != K.shape[2]:
        return O.attention(Q, K, V, dtype, scale) + 1.0
    return O.attention(Q, np.ascontiguousarray(K.transpose(0, 2, 1)), V, dtype, scale)


def mut_slices_mixed(Q, K, V, dtype, scale):
    # every slice attends to the keys and values of slice 0
    K0 = np.ascontiguousarray(np.repeat(K[:1], K.shape[0], axis=0))
    V0 = np.ascontiguousarray(np.repeat(V[:1], V.shape[0], axis=0))
    return O.attention(Q, K0, V0, dtype, scale)


def mut_exp_base_two(Q, K, V, dtype, scale):
    # exp2 in place of exp without the log2(e) factor folded into the scale
    return O.attention(Q, K, V, dtype, scale / math.log(2.0))


MUTANTS = [mut_no_max_subtraction, mut_no_normalisation, mut_softmax_over_queries, mut_scale_ignored,
           mut_scale_squared, mut_keys_as_values, mut_values_shifted, mut_last_key_dropped,
           mut_head_dim_transposed, mut_slices_mixed, mut_exp_base_two]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(oracle_mod, dtype, mutant):
    res = P.run_all(mutant, dtype)
    assert not all(res.values()), f"{mutant.__name__} passed every pin: {res}"
