"""Python binding of libswizzled_gemm.so (MI355X / gfx950 swizzled GEMM).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/swizzled_gemm.h``.  There is
no CPU fallback: if the shared library is missing, every call raises.

Two layers:

* ``gemm_run``, ``gemm_strided_run``, ``grouped_gemm_run``, ``mx_gemm_run``,
  ``mxfp4_gemm_run``, ``mxfp6_gemm_run``, ``gemm_layout_run``,
  ``gemm_layout128_run``, ``gemm_last_error``, ``gemm_version``,
  ``gemm_lds_layout``, ``gemm_lds_layout_mxfp6``, ``gemm_lds_layout_cblock``,
  ``gemm_lds_image``: the C entry points under the same names, taking integer
  device pointers.
* ``gemm``, ``gemm_strided``, ``grouped_gemm``, ``mx_gemm``, ``mxfp4_gemm``,
  ``mxfp6_gemm``, ``gemm_layout``, ``gemm_layout128``: the same calls on torch CUDA
  tensors (shapes read from the tensors, output allocated by torch, launched
  on torch's current stream).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "SG_OK", "SG_F16", "SG_BF16", "SG_F32", "SG_E4M3", "SG_E8M0", "SG_NONE",
    "SG_K_MAJOR", "SG_MN_MAJOR", "SG_MAX_GROUPS", "GemmError",
    "gemm_run", "gemm_strided_run", "grouped_gemm_run", "mx_gemm_run", "mxfp4_gemm_run",
    "mxfp6_gemm_run", "gemm_layout_run", "gemm_layout128_run", "gemm_last_error",
    "gemm_version", "gemm_lds_layout", "gemm_lds_layout_mxfp6", "gemm_lds_layout_cblock",
    "gemm_lds_image",
    "SG_E2M3", "SG_E3M2",
    "gemm", "gemm_plan", "gemm_strided", "grouped_gemm", "mx_gemm", "mxfp4_gemm", "mxfp6_gemm",
    "gemm_layout",
    "gemm_layout128", "SG_LAYOUT_PAD16",
    "library_path", "load",
]

SG_OK = 0
SG_NONE, SG_F16, SG_BF16, SG_F32, SG_E4M3, SG_E8M0 = 0, 1, 2, 3, 4, 5
SG_E2M3, SG_E3M2 = 7, 8
SG_K_MAJOR, SG_MN_MAJOR = 0, 1
SG_MAX_GROUPS = 128
SG_LAYOUT_PAD16 = -1
ERRORS = {-1: "SG_ERR_NULL", -2: "SG_ERR_ALIGN", -3: "SG_ERR_SHAPE",
          -4: "SG_ERR_DTYPE", -5: "SG_ERR_MAJOR", -6: "SG_ERR_GROUPS",
          -7: "SG_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libswizzled_gemm.so")
_lib = None


class GemmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.gemm_run.argtypes = [i64, i64, i64, vp, i32, vp, i32, i32, vp, i32, vp, i32, vp]
    f32 = ctypes.c_float
    lib.gemm_strided_run.argtypes = [i64, i64, i64, f32, vp, i64, i32, vp, i64, i32, i32,
                                     f32, vp, i64, i32, vp, i64, i32, vp]
    lib.grouped_gemm_run.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), i64, i64, vp,
                                     i32, vp, i32, i32, vp, i32, vp]
    lib.mx_gemm_run.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp]
    lib.mxfp4_gemm_run.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp]
    lib.mxfp6_gemm_run.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp]
    lib.gemm_layout_run.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, vp, i32, vp]
    lib.gemm_layout128_run.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, vp, i32, vp]
    lib.gemm_lds_layout.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_layout_mxfp6.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_layout_cblock.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_image.argtypes = [vp, i64, i64, i32, i64, i64, i32, vp, vp]
    for f in (lib.gemm_run, lib.gemm_strided_run, lib.grouped_gemm_run, lib.mx_gemm_run,
              lib.mxfp4_gemm_run, lib.mxfp6_gemm_run,
              lib.gemm_layout_run, lib.gemm_layout128_run,
              lib.gemm_lds_layout, lib.gemm_lds_layout_mxfp6, lib.gemm_lds_layout_cblock,
              lib.gemm_lds_image):
        f.restype = ctypes.c_int
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_version.argtypes = []
    lib.gemm_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ------------------------------------------------------------ raw C entry points

def gemm_run(M, N, K, A, a_major, B, b_major, ab_dtype, C, c_dtype, D, d_dtype,
             stream) -> int:
    return load().gemm_run(M, N, K, A, a_major, B, b_major, ab_dtype, C, c_dtype,
                           D, d_dtype, stream)


def gemm_strided_run(M, N, K, alpha, A, lda, a_major, B, ldb, b_major, ab_dtype, beta, C,
                     ldc, c_dtype, D, ldd, d_dtype, stream) -> int:
    return load().gemm_strided_run(M, N, K, alpha, A, lda, a_major, B, ldb, b_major,
                                   ab_dtype, beta, C, ldc, c_dtype, D, ldd, d_dtype, stream)


def grouped_gemm_run(G, m_offsets, N, K, A, a_major, B, b_major, ab_dtype, D,
                     d_dtype, stream) -> int:
    offs = None
    if m_offsets is not None:
        offs = (ctypes.c_int64 * len(m_offsets))(*[int(x) for x in m_offsets])
    return load().grouped_gemm_run(G, offs, N, K, A, a_major, B, b_major, ab_dtype,
                                   D, d_dtype, stream)


def mx_gemm_run(M, N, K, A, SFA, B, SFB, D, d_dtype, stream) -> int:
    return load().mx_gemm_run(M, N, K, A, SFA, B, SFB, D, d_dtype, stream)


def mxfp4_gemm_run(M, N, K, A, SFA, B, SFB, D, d_dtype, stream) -> int:
    return load().mxfp4_gemm_run(M, N, K, A, SFA, B, SFB, D, d_dtype, stream)


def mxfp6_gemm_run(fmt, M, N, K, A, SFA, B, SFB, D, d_dtype, stream) -> int:
    return load().mxfp6_gemm_run(fmt, M, N, K, A, SFA, B, SFB, D, d_dtype, stream)


def gemm_layout_run(swz_units, M, N, K, A, B, C, c_dtype, D, d_dtype, stream) -> int:
    return load().gemm_layout_run(swz_units, M, N, K, A, B, C, c_dtype, D, d_dtype, stream)


def gemm_layout128_run(layout, M, N, K, A, B, C, c_dtype, D, d_dtype, stream) -> int:
    return load().gemm_layout128_run(layout, M, N, K, A, B, C, c_dtype, D, d_dtype, stream)


def gemm_last_error() -> str:
    return load().gemm_last_error().decode()


def gemm_version() -> str:
    return load().gemm_version().decode()


def gemm_lds_layout(rows: int, row_bytes: int) -> np.ndarray:
    """[rows][row_bytes/16] LDS byte offsets of the kernels' swizzled tile."""
    out = np.zeros(max(rows, 0) * max(row_bytes // 16, 0) + 1, dtype=np.int32)
    rc = load().gemm_lds_layout(rows, row_bytes,
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != SG_OK:
        raise GemmError(rc, gemm_last_error())
    return out[:-1].reshape(rows, row_bytes // 16)


def gemm_lds_layout_mxfp6(rows: int, unshifted: int = 32) -> np.ndarray:
    """[rows][12] LDS byte offsets of bytes [8q, 8q+8) of each 96-byte row of
    the MXFP6 kernel's operand tile."""
    out = np.zeros(max(rows, 0) * 12 + 1, dtype=np.int32)
    rc = load().gemm_lds_layout_mxfp6(rows, unshifted,
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != SG_OK:
        raise GemmError(rc, gemm_last_error())
    return out[:-1].reshape(rows, 12)


def gemm_lds_layout_cblock() -> np.ndarray:
    """[4][128][8] LDS places of a 16-bit C in the 256x256 kernel's epilogue:
    wave, row and 16-byte chunk of the wave's 128 x 64 block -> quarter *
    16384 + byte offset inside that quarter's 16 KiB half slot."""
    out = np.zeros(4 * 128 * 8, dtype=np.int32)
    rc = load().gemm_lds_layout_cblock(out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != SG_OK:
        raise GemmError(rc, gemm_last_error())
    return out.reshape(4, 128, 8)


def gemm_lds_image(X, rows_total, K, elem_bytes, row0, k0, tile_rows, out,
                   stream) -> int:
    return load().gemm_lds_image(X, rows_total, K, elem_bytes, row0, k0, tile_rows,
                                 out, stream)


# ----------------------------------------------------------- torch convenience

def _check(rc: int):
    if rc != SG_OK:
        raise GemmError(rc, gemm_last_error())


def _dt(t) -> int:
    import torch
    m = {torch.float16: SG_F16, torch.bfloat16: SG_BF16, torch.float32: SG_F32}
    if t not in m:
        raise GemmError(-4, f"unsupported dtype {t}")
    return m[t]


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def gemm(A, B, *, a_major: str = "k", b_major: str = "k", C=None,
         out_dtype=None, out=None):
    """D = A*B (+C) on torch CUDA tensors.

    A: [M][K] (a_major "k") or [K][M] ("mn"); B: [N][K] ("k") or [K][N]
    ("mn"); C: optional [M][N]; returns D [M][N] of out_dtype (default
    torch.float32)."""
    import torch
    if a_major == "k":
        M, K = A.shape
    else:
        K, M = A.shape
    if b_major == "k":
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K or A.dtype != B.dtype:
        raise GemmError(-3, "A and B disagree on K or dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
    _check(gemm_run(M, N, K, A.data_ptr(), 0 if a_major == "k" else 1, B.data_ptr(),
                    0 if b_major == "k" else 1, _dt(A.dtype),
                    C.data_ptr() if C is not None else None,
                    _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                    _dt(out.dtype), _stream(A.device)))
    return out


def gemm_plan(A, B, *, a_major: str = "k", b_major: str = "k", C=None, out):
    """gemm() with its argument marshalling done once: returns a callable
    that launches D = A*B (+C) into `out` on the stream current now, for
    launch-bound small problems where the per-call Python work would
    otherwise take longer than the kernel.  The tensors must stay alive and
    keep their storage while the callable is in use."""
    if a_major == "k":
        M, K = A.shape
    else:
        K, M = A.shape
    if b_major == "k":
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K or A.dtype != B.dtype or tuple(out.shape) != (M, N):
        raise GemmError(-3, "A, B and out disagree on shapes or dtype")
    f = load().gemm_run
    args = (M, N, K, A.data_ptr(), 0 if a_major == "k" else 1, B.data_ptr(),
            0 if b_major == "k" else 1, _dt(A.dtype),
            C.data_ptr() if C is not None else None,
            _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(), _dt(out.dtype),
            _stream(A.device))

    def run() -> None:
        rc = f(*args)
        if rc != SG_OK:
            raise GemmError(rc, gemm_last_error())
    return run


def _ld(t, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise GemmError(-2, f"{name} must be 2-D with unit column stride")
    return t.stride(0)


def gemm_strided(A, B, *, a_major: str = "k", b_major: str = "k", C=None, alpha: float = 1.0,
                 beta: float = 1.0, out_dtype=None, out=None):
    """D = alpha * A*B + beta * C on 2-D torch CUDA tensors whose rows may be
    padded (views with unit column stride): leading dimensions are the row
    strides.  Shapes as in gemm(); `out` may itself be a padded view."""
    import torch
    if a_major == "k":
        M, K = A.shape
    else:
        K, M = A.shape
    if b_major == "k":
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K or A.dtype != B.dtype:
        raise GemmError(-3, "A and B disagree on K or dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
    _check(gemm_strided_run(M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"),
                            0 if a_major == "k" else 1, B.data_ptr(), _ld(B, "B"),
                            0 if b_major == "k" else 1, _dt(A.dtype), float(beta),
                            C.data_ptr() if C is not None else None,
                            _ld(C, "C") if C is not None else N,
                            _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                            _ld(out, "out"), _dt(out.dtype), _stream(A.device)))
    return out


def gemm_layout(A, B, swz_units: int, *, C=None, out_dtype=None, out=None):
    """gemm() for bf16 K-major A [M][K] and B [N][K] on the 256x256-tile
    kernel with the LDS layout swz_units (16 = the library's XOR swizzle
    over 256-byte lines, 8 = over 128-byte lines, 0 = none)."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
    _check(gemm_layout_run(swz_units, M, N, K, A.data_ptr(), B.data_ptr(),
                           C.data_ptr() if C is not None else None,
                           _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                           _dt(out.dtype), _stream(A.device)))
    return out


def grouped_gemm(A, B, m_offsets: Sequence[int], *, out_dtype=None, out=None):
    """Per group g: D[off_g:off_{g+1}] = A[off_g:off_{g+1}] * B[g]^T.

    A: [sum M][K]; B: [G][N][K]; m_offsets: G+1 host ints."""
    import torch
    G, N, K = B.shape
    if out is None:
        out = torch.empty((A.shape[0], N), dtype=out_dtype or torch.bfloat16,
                          device=A.device)
    _check(grouped_gemm_run(G, list(m_offsets), N, K, A.data_ptr(), 0, B.data_ptr(), 0,
                            _dt(A.dtype), out.data_ptr(), _dt(out.dtype),
                            _stream(A.device)))
    return out


def mx_gemm(A, SFA, B, SFB, *, out_dtype=None, out=None):
    """Block-scaled e4m3 GEMM: A [M][K], B [N][K] (uint8 e4m3 codes),
    SFA [M][K/32], SFB [N][K/32] (uint8 e8m0 codes)."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
    _check(mx_gemm_run(M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                       SFB.data_ptr(), out.data_ptr(), _dt(out.dtype),
                       _stream(A.device)))
    return out


def mxfp4_gemm(A, SFA, B, SFB, *, out_dtype=None, out=None):
    """Block-scaled e2m1 GEMM: A [M][K/2], B [N][K/2] (uint8, two e2m1 per
    byte, element 2i in the low nibble), SFA [M][K/32], SFB [N][K/32] (uint8
    e8m0 codes)."""
    import torch
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
    _check(mxfp4_gemm_run(M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                          SFB.data_ptr(), out.data_ptr(), _dt(out.dtype), _stream(A.device)))
    return out


def mxfp6_gemm(A, SFA, B, SFB, *, fmt: str = "e2m3", out_dtype=None, out=None):
    """Block-scaled FP6 GEMM: A [M][3K/4], B [N][3K/4] (uint8, a 6-bit
    stream of e2m3 or e3m2 codes per row, element k at bits [6k, 6k+6)),
    SFA [M][K/32], SFB [N][K/32] (uint8 e8m0 codes)."""
    import torch
    code = {"e2m3": SG_E2M3, "e3m2": SG_E3M2}[fmt]
    M, K = A.shape[0], A.shape[1] * 4 // 3
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
    _check(mxfp6_gemm_run(code, M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                          SFB.data_ptr(), out.data_ptr(), _dt(out.dtype), _stream(A.device)))
    return out


def gemm_layout128(A, B, layout: int, *, C=None, out_dtype=None, out=None):
    """gemm_layout() on 128x128 tiles, where layout may also be
    SG_LAYOUT_PAD16 (rows padded by 16 bytes, no swizzle)."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
    _check(gemm_layout128_run(layout, M, N, K, A.data_ptr(), B.data_ptr(),
                              C.data_ptr() if C is not None else None,
                              _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                              _dt(out.dtype), _stream(A.device)))
    return out
