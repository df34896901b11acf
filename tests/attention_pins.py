"""Pins for an attention implementation, checked against facts fixed outside it.

Every check takes ``attn(Q, K, V, dtype, scale) -> O`` with the calling
convention of ``oracle.oracle.attention`` (stored bit patterns, Q (BH, Sq, D),
K and V (BH, Sk, D), O float64 (BH, Sq, D)) and returns True when the
implementation reproduces a value that mathematics fixes independently of
the oracle's code: a pure-Python loop on tiny shapes, equal weights (a zero
query row, or queries orthogonal to every key) averaging the value rows, a
closed form for one-hot queries against a permutation of one-hot keys (the
weights are e^x and 1), the same closed form with logits of 1000 (where exp
overflows unless the row maximum is subtracted), the invariances of softmax
(a shift of every key by one vector, a joint permutation of keys and values)
and probabilities in place of the output when V is the identity.
"""
from __future__ import annotations

import math

import numpy as np

from software_pipelined_tiling_amd.inputs import draw, f64_to_f16_bits, f32_to_bf16_bits


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f64_to_f16_bits(x) if dtype == "f16" else f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _values(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _close(got, want, tol=1e-12) -> bool:
    got = np.asarray(got, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(want)))) if np.size(want) else 1.0
    return got.shape == np.shape(want) and bool(np.all(np.abs(got - want) <= tol * scale))


def pin_brute_force(attn, dtype: str, rng) -> bool:
    """Tiny shapes against a pure-Python loop over numpy-decoded values."""
    for BH, Sq, Sk, D in [(1, 1, 1, 1), (2, 3, 2, 4), (1, 4, 5, 3), (2, 2, 7, 2)]:
        Q = draw("uniform", -2, 2, (BH, Sq, D), rng, dtype)
        K = draw("uniform", -2, 2, (BH, Sk, D), rng, dtype)
        V = draw("uniform", -2, 2, (BH, Sk, D), rng, dtype)
        q, k, v = _values(Q, dtype), _values(K, dtype), _values(V, dtype)
        scale = 0.7
        want = np.zeros((BH, Sq, D))
        for b in range(BH):
            for i in range(Sq):
                s = [scale * sum(float(q[b, i, d]) * float(k[b, j, d]) for d in range(D)) for j in range(Sk)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(D):
                    want[b, i, d] = sum(e[j] / z * float(v[b, j, d]) for j in range(Sk))
        if not _close(attn(Q, K, V, dtype, scale), want):
            return False
    return True


def pin_equal_weights(attn, dtype: str, rng) -> bool:
    """A zero query row, or keys orthogonal to every query, weigh all keys alike:
    each output row is the mean of the value rows."""
    BH, Sq, Sk, D = 2, 5, 9, 8
    V = draw("uniform", -1, 1, (BH, Sk, D), rng, dtype)
    mean = _values(V, dtype).mean(axis=1)
    Q0 = _store(np.zeros((BH, Sq, D)), dtype)
    K = draw("uniform", -1, 1, (BH, Sk, D), rng, dtype)
    if not _close(attn(Q0, K, V, dtype, 1.0), np.repeat(mean[:, None, :], Sq, axis=1)):
        return False
    q = np.zeros((BH, Sq, D))
    q[:, :, : D // 2] = rng.integers(-3, 4, (BH, Sq, D // 2))
    k = np.zeros((BH, Sk, D))
    k[:, :, D // 2:] = rng.integers(-3, 4, (BH, Sk, D - D // 2))
    return _close(attn(_store(q, dtype), _store(k, dtype), V, dtype, 0.5), np.repeat(mean[:, None, :], Sq, axis=1))


def _soft_permutation(attn, dtype, rng, c, scale, n=16, D=16):
    """Q_i = c e_i, K_j = c e_{pi(j)}: row i scores x = scale c^2 on key j* = pi^-1(i)
    and 0 on the others, so O_i = (e^x V_j* + sum_{j != j*} V_j) / (e^x + n - 1),
    written as V_j* + (sum_{j != j*} (V_j - V_j*)) / (e^x + n - 1)."""
    pi = rng.permutation(n)
    q = np.zeros((1, n, D))
    q[0, np.arange(n), np.arange(n)] = c
    k = np.zeros((1, n, D))
    k[0, np.arange(n), pi] = c
    V = draw("uniform", -1, 1, (1, n, D), rng, dtype)
    v = _values(V, dtype)[0]
    x = scale * c * c
    inv = np.argsort(pi)
    want = np.empty((1, n, D))
    for i in range(n):
        js = inv[i]
        rest = np.delete(v, js, axis=0) - v[js]
        want[0, i] = v[js] + rest.sum(axis=0) / (math.exp(x) + n - 1) if x < 700 else v[js]
    return _close(attn(_store(q, dtype), _store(k, dtype), V, dtype, scale), want, 1e-12)


def pin_soft_permutation(attn, dtype: str, rng) -> bool:
    return all(_soft_permutation(attn, dtype, rng, 2.0, s) for s in (0.125, 0.75, 1.0, 2.5))


def pin_large_logits(attn, dtype: str, rng) -> bool:
    """Logits of 1000: exp overflows unless the row maximum is subtracted; the
    output is then the selected value row exactly (the others weigh e^-1000)."""
    return _soft_permutation(attn, dtype, rng, 2.0, 250.0)


def pin_invariances(attn, dtype: str, rng) -> bool:
    """Shifting every key by one vector changes row i's logits by one constant;
    permuting the keys and values together changes nothing."""
    BH, Sq, Sk, D = 2, 6, 11, 8
    q = rng.integers(-2, 3, (BH, Sq, D)).astype(np.float64)
    k = rng.integers(-2, 3, (BH, Sk, D)).astype(np.float64)
    V = draw("uniform", -1, 1, (BH, Sk, D), rng, dtype)
    base = attn(_store(q, dtype), _store(k, dtype), V, dtype, 0.25)
    shift = rng.integers(-2, 3, (BH, 1, D)).astype(np.float64)
    if not _close(attn(_store(q, dtype), _store(k + shift, dtype), V, dtype, 0.25), base, 1e-12):
        return False
    perm = rng.permutation(Sk)
    K2, V2 = _store(k[:, perm], dtype), np.ascontiguousarray(V[:, perm])
    return _close(attn(_store(q, dtype), K2, V2, dtype, 0.25), base, 1e-12)


def pin_identity_values(attn, dtype: str, rng) -> bool:
    """V = I (D = Sk): O is the probability matrix itself -- rows sum to one and
    log(O_ij / O_ik) = scale * Q_i . (K_j - K_k)."""
    BH, Sq, Sk = 1, 5, 8
    Q = draw("uniform", -1, 1, (BH, Sq, Sk), rng, dtype)
    K = draw("uniform", -1, 1, (BH, Sk, Sk), rng, dtype)
    V = _store(np.eye(Sk)[None], dtype)
    scale = 0.9
    P = np.asarray(attn(Q, K, V, dtype, scale))[0]
    q, k = _values(Q, dtype)[0], _values(K, dtype)[0]
    if not _close(P.sum(axis=1), np.ones(Sq)) or not np.all(P > 0):
        return False
    logit = scale * q @ k.T
    return _close(np.log(P[:, 1:] / P[:, :1]), logit[:, 1:] - logit[:, :1], 1e-10)


PINS = [pin_brute_force, pin_equal_weights, pin_soft_permutation, pin_large_logits, pin_invariances,
        pin_identity_values]


def run_all(attn, dtype: str) -> dict:
    out = {}
    for i, p in enumerate(PINS):
        try:
            out[p.__name__] = bool(p(attn, dtype, np.random.default_rng(1000 + i)))
        except (FloatingPointError, ValueError, OverflowError):
            out[p.__name__] = False
    return out
