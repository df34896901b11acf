"""Helpers for comparing the HIP path with the CPU oracle.

Float results: max |C_gpu - C_ref| / (||A[i,:]||_2 * ||B[:,j]||_2) <= tol, with
tol = 2e-3 for fp16 / bf16 inputs and 1e-5 for fp32 (fp32 accumulation);
where the norm product is zero C_gpu must be exactly zero.  int8 results
must be bit-exact.
"""
from __future__ import annotations

import numpy as np

TOL = {"f16": 2e-3, "bf16": 2e-3, "f32": 1e-5}


def values(bits: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of stored operands (numpy conversions)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.float64)


def logical_b(B: np.ndarray, b_col: bool, K: int, N: int) -> np.ndarray:
    return B[:N, :K].T if b_col else B[:K, :N]


def norm_products(A: np.ndarray, B: np.ndarray, dtype: str, b_col: bool, M: int, N: int, K: int):
    Av = values(np.ascontiguousarray(A[:M, :K]), dtype)
    Bv = values(np.ascontiguousarray(logical_b(B, b_col, K, N)), dtype)
    return np.linalg.norm(Av, axis=1), np.linalg.norm(Bv, axis=0)


def float_error(c_gpu: np.ndarray, c_ref: np.ndarray, rn: np.ndarray, cn: np.ndarray) -> float:
    """Max normalised error over the given outputs (rn, cn broadcast to c's shape)."""
    denom = rn * cn
    err = np.abs(c_gpu.astype(np.float64) - c_ref)
    zero = denom == 0
    if np.any(zero & (c_gpu != 0)):
        return float("inf")
    if not np.all(np.isfinite(c_gpu)):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, err / np.where(zero, 1.0, denom))
    return float(r.max()) if r.size else 0.0


def check_full(c_gpu, c_ref, A, B, dtype, b_col, M, N, K):
    """Raise AssertionError unless c_gpu matches the oracle's full product."""
    assert c_gpu.shape == c_ref.shape == (M, N)
    if dtype == "i8":
        bad = np.argwhere(c_gpu != c_ref)
        assert bad.size == 0, f"{len(bad)} int8 mismatches, first at {bad[:3].tolist()}"
        return 0.0
    rn, cn = norm_products(A, B, dtype, b_col, M, N, K)
    e = float_error(c_gpu, c_ref, rn[:, None], cn[None, :])
    assert e <= TOL[dtype], f"normalised error {e:.3e} > {TOL[dtype]:.1e}"
    return e


def check_entries(vals_gpu, vals_ref, rows, cols, A, B, dtype, b_col, M, N, K):
    if dtype == "i8":
        bad = np.flatnonzero(vals_gpu != vals_ref)
        assert bad.size == 0, f"{bad.size} int8 mismatches, first at {(rows[bad[:3]], cols[bad[:3]])}"
        return 0.0
    rn, cn = norm_products(A, B, dtype, b_col, M, N, K)
    e = float_error(vals_gpu, vals_ref, rn[rows], cn[cols])
    assert e <= TOL[dtype], f"normalised error {e:.3e} > {TOL[dtype]:.1e}"
    return e


def sample_entries(M: int, N: int, n: int, rng: np.random.Generator, BM: int = 128, BN: int = 256):
    """Random outputs plus every corner of every tile row/column edge and the matrix edges."""
    r = list(rng.integers(0, M, n))
    c = list(rng.integers(0, N, n))
    edge_r = sorted({0, M - 1} | {min(M - 1, k * BM + d) for k in range(0, M // BM + 1) for d in (0, BM - 1)})
    edge_c = sorted({0, N - 1} | {min(N - 1, k * BN + d) for k in range(0, N // BN + 1) for d in (0, BN - 1)})
    for i in edge_r[:: max(1, len(edge_r) // 16)]:
        for j in edge_c[:: max(1, len(edge_c) // 16)]:
            r.append(i)
            c.append(j)
    return np.array(r, dtype=np.int64), np.array(c, dtype=np.int64)


# Attention: O_gpu - O_ref at (b, i, d), over max_j |V[b, j, d]|.  The softmax weights of a
# row sum to one, so |O[b, i, d]| <= max_j |V[b, j, d]|: this is the scale of every output
# in column d.  The kernel rounds each probability to the input type (relative error at
# most u = 2^-8 for bf16, 2^-11 for fp16) and divides by the sum of the rounded values,
# so its weights are w_j (1 + e_j) / (1 + sum_k w_k e_k): the output moves by
# sum_j w_j e_j (V_j - O) / (1 + ...), at most 2u / (1 - u) times max_j |V[b, j, d]|
# (7.84e-3 for bf16, 9.8e-4 for fp16); fp32 sums add far less.
TOL_ATTN = {"f16": 2e-3, "bf16": 8e-3}


def attention_error(o_gpu, o_ref, v_bits, dtype) -> float:
    v = values(np.ascontiguousarray(v_bits), dtype)           # (BH, Sk, D)
    scale = np.max(np.abs(v), axis=1, keepdims=True)           # (BH, 1, D)
    if not np.all(np.isfinite(o_gpu)):
        return float("inf")
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    zero = scale == 0
    if np.any(np.broadcast_to(zero, err.shape) & (o_gpu != 0)):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, err / np.where(zero, 1.0, scale))
    return float(r.max()) if r.size else 0.0


def check_attention(o_gpu, o_ref, v_bits, dtype) -> float:
    e = attention_error(o_gpu, o_ref, v_bits, dtype)
    assert e <= TOL_ATTN[dtype], f"attention normalised error {e:.3e} > {TOL_ATTN[dtype]:.1e}"
    return e
