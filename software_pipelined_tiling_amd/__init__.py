"""software_pipelined_tiling_amd -- software-pipelined tiled GEMM for AMD MI355X (gfx950).

Thin ctypes binding of ``libspt.so`` (C ABI in ``include/spt.h``).  The
functions ``spt_gemm``, ``spt_gemm_ex``, ``spt_plan``, ``spt_status_string``,
``spt_last_error`` and ``spt_version`` keep the C names and arguments (device
pointers as Python ints, ``stream`` as a hipStream_t handle or 0).  ``gemm``
is a convenience wrapper for torch tensors that only marshals arguments:
every step of the product runs in the library's HIP kernels, and there is no
other code path -- if ``libspt.so`` cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "spt_gemm", "spt_gemm_ex", "spt_plan", "spt_status_string", "spt_last_error", "spt_version",
    "spt_scale_by_two", "spt_attention", "attention", "gemm", "plan", "scale_by_two", "SptError", "PlanInfo", "lib_path",
    "F16", "BF16", "I8", "F32", "ROW", "COL", "VARIANT_AUTO", "VARIANT_SYNC", "VARIANT_REG",
    "VARIANT_DIRECT", "VARIANT_PERSIST", "TILE_AUTO", "TILE_128x256", "TILE_256x256", "TILE_128x128", "TILE_256x256_4W",
    "TILE_256x256_4W_K64B", "TILE_256x192",
]

HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(HERE, "libspt.so")

# enum spt_dtype / spt_layout / spt_variant / spt_tile / spt_status
F16, BF16, I8, F32 = 0, 1, 2, 3
ROW, COL = 0, 1
VARIANT_AUTO, VARIANT_SYNC, VARIANT_REG, VARIANT_DIRECT, VARIANT_PERSIST = 0, 1, 2, 3, 4
TILE_AUTO, TILE_128x256, TILE_256x256, TILE_128x128, TILE_256x256_4W, TILE_256x256_4W_K64B, TILE_256x192 = (
    0, 1, 2, 3, 4, 5, 6)
SPT_OK, SPT_ERR_INVALID, SPT_ERR_UNSUPPORTED, SPT_ERR_MISALIGNED, SPT_ERR_LAUNCH = 0, -1, -2, -3, -4

DTYPE_CODES = {"f16": F16, "bf16": BF16, "i8": I8, "f32": F32}
VARIANT_CODES = {"auto": VARIANT_AUTO, "sync": VARIANT_SYNC, "reg": VARIANT_REG, "direct": VARIANT_DIRECT,
                 "persist": VARIANT_PERSIST}


class PlanInfo(ctypes.Structure):
    """Mirror of ``spt_plan_info``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("b_layout", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("stages", ctypes.c_int32), ("tile_id", ctypes.c_int32),
        ("BM", ctypes.c_int32), ("BN", ctypes.c_int32), ("BK", ctypes.c_int32),
        ("threads", ctypes.c_int32), ("waves", ctypes.c_int32),
        ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32), ("elt_bytes", ctypes.c_int32),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("grid", ctypes.c_int64),
        ("k_tiles", ctypes.c_int64), ("k_full_tiles", ctypes.c_int64), ("k_tail", ctypes.c_int32),
        ("a_stage_bytes", ctypes.c_int32), ("b_stage_bytes", ctypes.c_int32),
        ("stage_bytes", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("a_copies_per_thread", ctypes.c_int32), ("b_copies_per_thread", ctypes.c_int32),
        ("wg_per_cu_lds", ctypes.c_int32), ("waves_per_simd_lds", ctypes.c_int32),
        ("steady_vmcnt", ctypes.c_int32), ("mfma_per_ktile_per_wave", ctypes.c_int32),
        ("ratio_flop_per_byte", ctypes.c_double), ("ratio_mfma_per_load", ctypes.c_double),
        ("store_window", ctypes.c_int32), ("tiles_per_wg", ctypes.c_int32),
        ("band_tile", ctypes.c_int32), ("band_stages", ctypes.c_int32), ("band_m", ctypes.c_int64), ("band_grid", ctypes.c_int64),
        ("tail_ring", ctypes.c_int32), ("half_stage_slots", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class SptError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {spt_status_string(status)} ({spt_last_error()})")


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"libspt.so not found at {lib_path}: build it with "
                               "`python -m software_pipelined_tiling_amd.build`")
        L = ctypes.CDLL(lib_path)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.spt_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp]
        L.spt_gemm.restype = i32
        L.spt_gemm_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp, i32, i32, i32, i32]
        L.spt_gemm_ex.restype = i32
        L.spt_plan.argtypes = [i32, i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(PlanInfo)]
        L.spt_plan.restype = i32
        L.spt_status_string.argtypes = [i32]
        L.spt_status_string.restype = ctypes.c_char_p
        L.spt_last_error.argtypes = []
        L.spt_last_error.restype = ctypes.c_char_p
        L.spt_version.argtypes = []
        L.spt_version.restype = i32
        L.spt_scale_by_two.argtypes = [i64, vp, vp, i32, i32, vp]
        L.spt_scale_by_two.restype = i32
        L.spt_attention.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, i32, vp, i32, i32]
        L.spt_attention.restype = i32
        _lib = L
    return _lib


def lib() -> ctypes.CDLL:
    """The loaded ``libspt.so`` (raises if it is missing)."""
    return _load()


# ---- the C ABI, same names ---------------------------------------------------

def spt_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=0) -> int:
    return _load().spt_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream)


def spt_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream, b_layout, variant, stages,
                tile_id) -> int:
    return _load().spt_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream, b_layout, variant,
                               stages, tile_id)


def spt_plan(dtype, M, N, K, b_layout=ROW, variant=VARIANT_AUTO, stages=0, tile_id=TILE_AUTO):
    """Returns (status, PlanInfo)."""
    info = PlanInfo()
    rc = _load().spt_plan(dtype, M, N, K, b_layout, variant, stages, tile_id, ctypes.byref(info))
    return rc, info


def spt_scale_by_two(n, x, y, stages=0, blocks=0, stream=0) -> int:
    return _load().spt_scale_by_two(n, x, y, stages, blocks, stream)


def spt_attention(BH, Sq, Sk, D, Q, K, V, O, scale, dtype, stream=0, variant=VARIANT_AUTO, stages=0) -> int:
    return _load().spt_attention(BH, Sq, Sk, D, Q, K, V, O, scale, dtype, stream, variant, stages)


def spt_status_string(status: int) -> str:
    return _load().spt_status_string(status).decode()


def spt_last_error() -> str:
    return _load().spt_last_error().decode()


def spt_version() -> int:
    return _load().spt_version()


# ---- torch convenience ---------------------------------------------------------

def _torch_dtype_code(t):
    import torch
    m = {torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8, torch.float32: F32}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def plan(dtype: str | int, M: int, N: int, K: int, *, b_layout: str = "row", variant: str = "auto",
         stages: int = 0, tile: int = 0) -> dict:
    d = DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype
    rc, info = spt_plan(d, M, N, K, COL if b_layout == "col" else ROW, VARIANT_CODES[variant],
                        stages, tile)
    if rc != SPT_OK:
        raise SptError(rc, "spt_plan")
    return info.as_dict()


def gemm(A, B, out=None, *, b_layout: str = "row", variant: str = "auto", stages: int = 0,
         tile: int = 0, stream=None, K: int | None = None, N: int | None = None):
    """C = A @ B for torch tensors on the GPU, through ``spt_gemm_ex``.

    A: (M, >=K) with unit column stride (row pitch = A.stride(0)).
    B: row-major (K, >=N) or, with b_layout='col', (N, >=K) holding B^T.
    out: (M, >=N) float32 (int32 for int8 inputs); allocated when None.
    K / N default to the operand widths; pass them to treat the rest of each
    row as padding.
    """
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    d = _torch_dtype_code(A)
    if A.dim() != 2 or B.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B must be 2-D with unit column stride")
    if not A.is_cuda or B.device != A.device:
        raise ValueError("A and B must be on the same GPU")
    if b_layout not in ("row", "col"):
        raise ValueError("b_layout must be 'row' or 'col'")
    col = b_layout == "col"
    M = A.shape[0]
    K = A.shape[1] if K is None else K
    if N is None:
        N = B.shape[0] if col else B.shape[1]
    # the kernels read K columns of A and K x N of B: both must lie inside the tensors
    b_k, b_n = (B.shape[1], B.shape[0]) if col else (B.shape[0], B.shape[1])
    if not (0 <= K <= A.shape[1] and K <= b_k and 0 <= N <= b_n):
        raise ValueError(f"K={K}, N={N} exceed the operands A {tuple(A.shape)}, B {tuple(B.shape)}")
    c_dtype = torch.int32 if d == I8 else torch.float32
    if out is None:  # row pitch padded to 16 bytes; the result is the (M, N) view
        ldc = -(-max(N, 1) // 4) * 4
        out = torch.empty((M, ldc), dtype=c_dtype, device=A.device)[:, :N]
    if out.dtype != c_dtype or out.device != A.device:
        raise TypeError(f"out must be {c_dtype} on {A.device}")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] < N:
        raise ValueError("out must be (M, >=N) with unit column stride")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    with torch.cuda.device(A.device):  # the library launches on the calling thread's current device
        rc = spt_gemm_ex(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), out.data_ptr(),
                         out.stride(0), d, stream, COL if col else ROW, VARIANT_CODES[variant], stages,
                         tile)
    if rc != SPT_OK:
        raise SptError(rc, "spt_gemm_ex")
    return out


def attention(Q, K, V, scale: float | None = None, out=None, *, variant: str = "auto", stages: int = 0,
              stream=None):
    """O = softmax(scale * Q K^T) V for contiguous fp16/bf16 torch tensors on the GPU
    (Q (BH, Sq, D), K and V (BH, Sk, D)), through ``spt_attention``; O is fp32.
    `scale` defaults to 1/sqrt(D)."""
    import torch
    if Q.dtype != K.dtype or Q.dtype != V.dtype or Q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("Q, K, V must share one dtype, float16 or bfloat16")
    if Q.dim() != 3 or K.dim() != 3 or K.shape != V.shape or K.shape[0] != Q.shape[0] or K.shape[2] != Q.shape[2]:
        raise ValueError("Q (BH, Sq, D), K and V (BH, Sk, D) expected")
    if not (Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()):
        raise ValueError("Q, K, V must be contiguous")
    if not Q.is_cuda or K.device != Q.device or V.device != Q.device:
        raise ValueError("Q, K, V must be on the same GPU")
    BH, Sq, D = Q.shape
    Sk = K.shape[1]
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((BH, Sq, D), dtype=torch.float32, device=Q.device)
    if out.dtype != torch.float32 or out.shape != (BH, Sq, D) or not out.is_contiguous() or out.device != Q.device:
        raise ValueError("out must be a contiguous float32 (BH, Sq, D) tensor on Q's GPU")
    if stream is None:
        stream = torch.cuda.current_stream(Q.device).cuda_stream
    with torch.cuda.device(Q.device):
        rc = spt_attention(BH, Sq, Sk, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), scale,
                           _torch_dtype_code(Q), stream, VARIANT_CODES[variant], stages)
    if rc != SPT_OK:
        raise SptError(rc, "spt_attention")
    return out


def scale_by_two(x, out=None, *, stages: int = 0, blocks: int = 0, stream=None):
    """out = 2 * x for a contiguous float32 torch tensor on the GPU, through
    ``spt_scale_by_two`` (out may be x itself)."""
    import torch
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    if not x.is_cuda:
        raise ValueError("x must be on the GPU")
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != x.numel():
        raise ValueError("out must be a contiguous float32 tensor of x's size")
    if out.device != x.device:
        raise ValueError("out must be on x's GPU")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = spt_scale_by_two(x.numel(), x.data_ptr(), out.data_ptr(), stages, blocks, stream)
    if rc != SPT_OK:
        raise SptError(rc, "spt_scale_by_two")
    return out
