"""Python face of the CPU oracle (``oracle.c``) for the tiled GEMM C = A*B
and the attention-style consumer O = softmax(scale Q K^T) V.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module; the HIP library and its
Python binding never import it, and it imports nothing from them.

The arithmetic lives in ``oracle.c`` (one k-ordered dot product per output,
in double for float inputs and int32 for int8 inputs -- the plain definition
of the product that "Pipeline GPU Kernel" (Schritt 5) says every pipelined
variant must reproduce).  This module only marshals numpy arrays into it.

Array conventions: float inputs are passed as their stored bit patterns
(``uint16`` for binary16 / bfloat16, ``uint32`` or ``float32`` for binary32);
int8 inputs as ``int8``.  ``A`` is a 2-D array whose rows are the M rows of
A (the array may be wider than K: its row pitch is lda).  ``B`` is a 2-D
array holding B row-major (K rows of pitch ldb) or, with ``b_col=True``,
column-major (N rows of pitch ldb, element (k, j) at ``B[j, k]``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DT_F16, DT_BF16, DT_F32 = 0, 1, 3
_DTYPES = {"f16": DT_F16, "bf16": DT_BF16, "f32": DT_F32}

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc + OpenMP into ``liboracle.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        # -ffp-contract=off: every product is rounded before it is added, as the
        # definition is written out, whatever the compiler's default target
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp,
                        SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIB)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.oracle_gemm_float.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, i32, vp, i64, i32]
        L.oracle_gemm_float_entries.argtypes = [i32, i64, vp, i64, vp, i64, i32, i64, vp, vp, vp, i32]
        L.oracle_gemm_int8.argtypes = [i64, i64, i64, vp, i64, vp, i64, i32, vp, i64, i32]
        L.oracle_gemm_int8_entries.argtypes = [i64, vp, i64, vp, i64, i32, i64, vp, vp, vp, i32]
        L.oracle_decode_array.argtypes = [i32, vp, i64, vp]
        L.oracle_max_threads.argtypes = []
        L.oracle_scale_by_two.argtypes = [i64, vp, vp]
        L.oracle_attention.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, ctypes.c_double, vp, i32]
        L.oracle_attention_rows.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, ctypes.c_double, i64, vp, vp,
                                            vp, i32]
        for f in ("oracle_gemm_float", "oracle_gemm_float_entries", "oracle_gemm_int8",
                  "oracle_gemm_int8_entries", "oracle_decode_array", "oracle_max_threads", "oracle_attention",
                  "oracle_attention_rows"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc == -2:
        raise ValueError("oracle: int8 K too large for an exact int32 sum")
    if rc != 0:
        raise ValueError(f"oracle: invalid argument (rc={rc})")


def _as_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32" and x.dtype == np.float32:
        x = x.view(np.uint32)
    want = np.uint32 if dtype == "f32" else np.uint16
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be stored as {want.__name__}, got {x.dtype}")
    return np.ascontiguousarray(x)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decode of stored float values (binary16/bfloat16/binary32) into float64."""
    b = _as_bits(np.asarray(bits), dtype)
    out = np.empty(b.shape, dtype=np.float64)
    _check(lib().oracle_decode_array(_DTYPES[dtype], _ptr(b), b.size, _ptr(out)))
    return out


def _dims(A, B, b_col, K, N=None):
    M = A.shape[0]
    if N is None:
        N = B.shape[0] if b_col else B.shape[1]
    if K is None:
        K = A.shape[1]
    return M, N, K, A.shape[1], B.shape[1]


def gemm(A: np.ndarray, B: np.ndarray, dtype: str, *, b_col: bool = False, K: int | None = None,
         N: int | None = None, threads: int = 0) -> np.ndarray:
    """Full product.  Float dtypes return float64 (M, N); 'i8' returns int32 (M, N).

    ``K`` defaults to A's width and ``N`` to B's width (row-major B) or row
    count (column-major B); pass them to treat the remaining columns of each
    row as padding (the row pitch is the array's width).
    """
    M, N, K, lda, ldb = _dims(A, B, b_col, K, N)
    if dtype == "i8":
        A8 = np.ascontiguousarray(A, dtype=np.int8)
        B8 = np.ascontiguousarray(B, dtype=np.int8)
        C = np.zeros((M, N), dtype=np.int32)
        _check(lib().oracle_gemm_int8(M, N, K, _ptr(A8), lda, _ptr(B8), ldb, int(b_col), _ptr(C),
                                      max(N, 1), threads))
        return C
    Ab, Bb = _as_bits(A, dtype), _as_bits(B, dtype)
    C = np.zeros((M, N), dtype=np.float64)
    _check(lib().oracle_gemm_float(_DTYPES[dtype], M, N, K, _ptr(Ab), lda, _ptr(Bb), ldb,
                                   int(b_col), _ptr(C), max(N, 1), threads))
    return C


def gemm_entries(A: np.ndarray, B: np.ndarray, dtype: str, rows, cols, *, b_col: bool = False,
                 K: int | None = None, threads: int = 0) -> np.ndarray:
    """C[rows[e], cols[e]] for each e, each a separate k-ordered dot product."""
    _, _, K, lda, ldb = _dims(A, B, b_col, K)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows and cols must have the same shape")
    nrows = A.shape[0]
    ncols = B.shape[0] if b_col else B.shape[1]
    if r.size and (r.min() < 0 or r.max() >= nrows or c.min() < 0 or c.max() >= ncols):
        raise ValueError("entry index out of range")
    if dtype == "i8":
        A8 = np.ascontiguousarray(A, dtype=np.int8)
        B8 = np.ascontiguousarray(B, dtype=np.int8)
        out = np.zeros(r.shape, dtype=np.int32)
        _check(lib().oracle_gemm_int8_entries(K, _ptr(A8), lda, _ptr(B8), ldb, int(b_col), r.size,
                                              _ptr(r), _ptr(c), _ptr(out), threads))
        return out
    Ab, Bb = _as_bits(A, dtype), _as_bits(B, dtype)
    out = np.zeros(r.shape, dtype=np.float64)
    _check(lib().oracle_gemm_float_entries(_DTYPES[dtype], K, _ptr(Ab), lda, _ptr(Bb), ldb,
                                           int(b_col), r.size, _ptr(r), _ptr(c), _ptr(out),
                                           threads))
    return out


def scale_by_two(x: np.ndarray) -> np.ndarray:
    """y = 2 * x elementwise for a float32 vector ("Hiding Memory Latency ...",
    section 8); returns a new float32 array."""
    xb = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    y = np.empty_like(xb)
    _check(lib().oracle_scale_by_two(xb.size, _ptr(xb), _ptr(y)))
    return y.view(np.float32)


def _qkv(Q, K, V, dtype):
    if dtype not in ("f16", "bf16"):
        raise TypeError("oracle: attention inputs are f16 or bf16")
    Qb, Kb, Vb = (_as_bits(np.asarray(x), dtype) for x in (Q, K, V))
    if Qb.ndim != 3 or Kb.ndim != 3 or Kb.shape != Vb.shape or Qb.shape[0] != Kb.shape[0] or Qb.shape[2] != Kb.shape[2]:
        raise ValueError("oracle: Q (BH, Sq, D), K and V (BH, Sk, D) expected")
    return Qb, Kb, Vb


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str, scale: float,
              threads: int = 0) -> np.ndarray:
    """O = softmax(scale * Q K^T) V for each (batch, head) slice, in float64.

    Q (BH, Sq, D), K and V (BH, Sk, D), stored bit patterns of ``dtype``
    ('f16' or 'bf16'); returns O (BH, Sq, D) float64."""
    Qb, Kb, Vb = _qkv(Q, K, V, dtype)
    BH, Sq, D = Qb.shape
    O = np.zeros((BH, Sq, D), dtype=np.float64)
    _check(lib().oracle_attention(_DTYPES[dtype], BH, Sq, Kb.shape[1], D, _ptr(Qb), _ptr(Kb), _ptr(Vb),
                                  float(scale), _ptr(O), threads))
    return O


def attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str, scale: float, slices, rows,
                   threads: int = 0) -> np.ndarray:
    """O[slices[e], rows[e], :] for each e (same definition as ``attention``)."""
    Qb, Kb, Vb = _qkv(Q, K, V, dtype)
    BH, Sq, D = Qb.shape
    sl = np.ascontiguousarray(slices, dtype=np.int64)
    rw = np.ascontiguousarray(rows, dtype=np.int64)
    if sl.shape != rw.shape or sl.ndim != 1:
        raise ValueError("slices and rows must be 1-D of the same length")
    out = np.zeros((sl.size, D), dtype=np.float64)
    _check(lib().oracle_attention_rows(_DTYPES[dtype], BH, Sq, Kb.shape[1], D, _ptr(Qb), _ptr(Kb), _ptr(Vb),
                                       float(scale), sl.size, _ptr(sl), _ptr(rw), _ptr(out), threads))
    return out


def max_threads() -> int:
    return int(lib().oracle_max_threads())
