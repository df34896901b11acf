"""Seeded synthetic operands for the GEMM workloads (host numpy only).

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds none of the GEMM's arithmetic: it only draws random
values, rounds them to the storage format and lays them out.

Values are returned as their stored bit patterns: ``uint16`` for binary16 and
bfloat16, ``float32`` for binary32 and ``int8`` for int8.  Rounding to the
16-bit formats is round-to-nearest-even.

Generator: ``numpy.random.default_rng([workload_id, operand, K])`` with
operand 0 for A and 1 for B, so every operand of every workload has its own
reproducible stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ELT_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "i8": 1}
OUT_BYTES = {"f16": 4, "bf16": 4, "f32": 4, "i8": 4}


def rng_for(workload_id: int, operand: int, K: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(operand), int(K)])


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round to binary16 (numpy's cast is round-to-nearest-even) and return the bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 with round-to-nearest-even; return the bits.

    Finite inputs only (the generators never produce NaN).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def draw(dist: str, lo: float, hi: float, shape, rng: np.random.Generator, dtype: str) -> np.ndarray:
    """Draw ``shape`` values from ``dist`` and store them in ``dtype``."""
    if dtype == "i8":
        return rng.integers(int(lo), int(hi) + 1, size=shape, dtype=np.int16).astype(np.int8)
    if dist == "uniform":
        x = rng.uniform(lo, hi, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "intgrid":  # integers in [lo, hi], stored exactly in any float format
        x = rng.integers(int(lo), int(hi) + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(dist)
    if dtype == "f16":
        return f64_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    if dtype == "f32":
        return x.astype(np.float32)
    raise ValueError(dtype)


@dataclass(frozen=True)
class Workload:
    """One GEMM problem: sizes, storage, value distribution and seed."""
    name: str
    wid: int
    dtype: str
    M: int
    N: int
    K: int
    b_col: bool = False
    dist: str = "uniform"
    lo: float = -1.0
    hi: float = 1.0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> int:
        """Each operand read once, C written once."""
        e = ELT_BYTES[self.dtype]
        return e * self.M * self.K + e * self.K * self.N + OUT_BYTES[self.dtype] * self.M * self.N


def make_operands(w: Workload, lda: int | None = None, ldb: int | None = None):
    """Return (A, B) host arrays for workload ``w``.

    A has shape (M, lda) -- the first K columns hold the operand, padding
    columns hold zeros.  B has shape (K, ldb) row-major or (N, ldb) for a
    column-major B (``w.b_col``), first N (resp. K) columns used.
    """
    lda = w.K if lda is None else lda
    a = draw(w.dist, w.lo, w.hi, (w.M, w.K), rng_for(w.wid, 0, w.K), w.dtype)
    bshape = (w.N, w.K) if w.b_col else (w.K, w.N)
    b = draw(w.dist, w.lo, w.hi, bshape, rng_for(w.wid, 1, w.K), w.dtype)
    ldb = bshape[1] if ldb is None else ldb
    A = np.zeros((w.M, lda), dtype=a.dtype)
    A[:, : w.K] = a
    B = np.zeros((bshape[0], ldb), dtype=b.dtype)
    B[:, : bshape[1]] = b
    return A, B


# The five workloads of the headline measurement, with their seeds.
W_F16_256 = Workload("fp16 GEMM 256x256x256", 1, "f16", 256, 256, 256)
W_F16_4096 = Workload("fp16 GEMM 4096x4096x4096", 2, "f16", 4096, 4096, 4096)
W_I8_4096 = Workload("int8 GEMM 4096x4096x4096, B column-major", 3, "i8", 4096, 4096, 4096,
                     b_col=True, lo=-128, hi=127)


def w_bf16_lowk(K: int) -> Workload:
    return Workload(f"bf16 GEMM 8192x8192x{K} (low K)", 4, "bf16", 8192, 8192, K, dist="normal")


W_BF16_RAGGED = Workload("bf16 GEMM 4000x3000x1000 (ragged)", 5, "bf16", 4000, 3000, 1000,
                         lo=-2.0, hi=2.0)
LOWK_KS = (64, 128, 256, 512)


def scaled(w: Workload, M: int, N: int, K: int, wid: int | None = None) -> Workload:
    """Same dtype / layout / distribution at other sizes (for oracle-sized parity runs)."""
    return Workload(f"{w.name} @ {M}x{N}x{K}", w.wid if wid is None else wid, w.dtype, M, N, K,
                    w.b_col, w.dist, w.lo, w.hi)


@dataclass(frozen=True)
class AttentionWorkload:
    """One attention problem: BH (batch x heads) slices of Sq queries and Sk keys
    of head dimension D, entries drawn from `dist` and stored in `dtype`."""
    name: str
    wid: int
    BH: int
    Sq: int
    Sk: int
    D: int
    dtype: str = "f16"
    dist: str = "normal"
    lo: float = -1.0
    hi: float = 1.0

    @property
    def flops(self) -> int:
        """The two products, 4 * BH * Sq * Sk * D ("Kernel-Engpass analysieren", Schritt 1)."""
        return 4 * self.BH * self.Sq * self.Sk * self.D

    @property
    def alg_bytes(self) -> int:
        """Q, K and V read once, the fp32 output written once."""
        e = ELT_BYTES[self.dtype]
        return e * self.BH * self.D * (self.Sq + 2 * self.Sk) + 4 * self.BH * self.Sq * self.D


def make_qkv(w: AttentionWorkload):
    """(Q, K, V) host arrays of stored bits: Q (BH, Sq, D), K and V (BH, Sk, D)."""
    q = draw(w.dist, w.lo, w.hi, (w.BH, w.Sq, w.D), rng_for(w.wid, 0, w.Sk), w.dtype)
    k = draw(w.dist, w.lo, w.hi, (w.BH, w.Sk, w.D), rng_for(w.wid, 1, w.Sk), w.dtype)
    v = draw(w.dist, w.lo, w.hi, (w.BH, w.Sk, w.D), rng_for(w.wid, 2, w.Sk), w.dtype)
    return q, k, v


# The attention-style consumer: batch 2 x 16 heads, 4096 queries and keys, head
# dimension 128, N(0, 1) entries in fp16 (a flash-attention forward shape).
W_ATTN_4096 = AttentionWorkload("fp16 attention 32 x 4096 x 4096 x 128", 6, 32, 4096, 4096, 128)
