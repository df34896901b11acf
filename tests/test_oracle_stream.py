"""Pins of the streaming oracle y = 2 x ("Hiding Memory Latency ...", section 8).

Each pin fixes the result by something other than the oracle itself: the
pages' worked example (its input formula and the max_error it prints), a
closed form computed with integers, IEEE special values, and numpy's float32
multiply (a library routine).  Planted mistakes must each break a pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_stream_example.json")))


def pages_input(n):
    return ((np.arange(n, dtype=np.int64) % 113).astype(np.float32) * np.float32(0.25))


def pin_pages_example(f) -> bool:
    """The pages' example: max |y - 2 x| is 0, and y = (i mod 113) / 2 exactly."""
    n = GOLDEN["n"]
    x = pages_input(n)
    y = f(x)
    closed = (np.arange(n, dtype=np.int64) % 113).astype(np.float64) / 2.0
    err = float(np.max(np.abs(y.astype(np.float64) - 2.0 * x.astype(np.float64))))
    return y.shape == (n,) and err == GOLDEN["printed_max_error"] and np.array_equal(y.astype(np.float64), closed)


SPECIAL = [(0.0, 0.0), (-0.0, -0.0), (1.0, 2.0), (-3.5, -7.0), (np.inf, np.inf), (-np.inf, -np.inf),
           (3.4028234663852886e38, np.inf), (2.0 ** 127, np.inf),
           ((2.0 - 2.0 ** -23) * 2.0 ** 126, 3.4028234663852886e38),
           (1.401298464324817e-45, 2.802596928649634e-45), (1.1754942106924411e-38, 2.3509884213848822e-38)]


def pin_special_values(f) -> bool:
    """Signed zeros, infinities, overflow to infinity, the largest finite result,
    subnormals and the smallest normal: all exact."""
    x = np.array([a for a, _ in SPECIAL], dtype=np.float32)
    want = np.array([b for _, b in SPECIAL], dtype=np.float32)
    y = f(x)
    return np.array_equal(y.view(np.uint32), want.view(np.uint32)) and bool(np.isnan(f(np.array([np.nan], np.float32)))[0])


def pin_numpy_multiply(f) -> bool:
    """Random finite floats over the whole exponent range: bit-equal to numpy's float32 2 * x."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=100003, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    return np.array_equal(f(x).view(np.uint32), (np.float32(2.0) * x).view(np.uint32))


def pin_lengths(f) -> bool:
    """Every length from 0 to 9: the output has that length and every element is doubled."""
    for n in range(10):
        x = np.arange(1, n + 1, dtype=np.float32)
        y = f(x)
        if y.shape != (n,) or not np.array_equal(y, x * 2):
            return False
    return True


PINS = [pin_pages_example, pin_special_values, pin_numpy_multiply, pin_lengths]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(O.scale_by_two)


# ---- planted mistakes --------------------------------------------------------
def mut_copy(x):            # forgot the factor
    return np.ascontiguousarray(x, dtype=np.float32).copy()


def mut_drop_last(x):       # loop bound one short
    y = O.scale_by_two(x)
    if y.size:
        y[-1] = x[-1]
    return y


def mut_add_instead(x):     # 2 + x instead of 2 * x
    return (np.float32(2.0) + np.asarray(x, np.float32)).astype(np.float32)


def mut_shift(x):           # y[i] = 2 x[i+1]
    y = O.scale_by_two(x)
    return np.roll(y, -1) if y.size > 1 else y


def mut_flush_subnormal(x):  # subnormals flushed to zero
    y = O.scale_by_two(x)
    y[np.abs(np.asarray(x, np.float32)) < np.float32(1.1754942e-38)] = 0.0
    return y


def mut_via_half(x):        # computed in fp16
    return (np.asarray(x, np.float32).astype(np.float16) * np.float16(2)).astype(np.float32)


@pytest.mark.parametrize("mut", [mut_copy, mut_drop_last, mut_add_instead, mut_shift, mut_flush_subnormal,
                                 mut_via_half], ids=lambda m: m.__name__)
def test_pins_catch_planted_mistake(mut):
    with np.errstate(all="ignore"):
        assert not all(p(mut) for p in PINS)
