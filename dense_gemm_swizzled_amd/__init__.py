"""Python binding of libswizzled_gemm.so (MI355X / gfx950 swizzled GEMM).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/swizzled_gemm.h``.  There is
no CPU fallback: if the shared library is missing, every call raises.

Two layers:

* ``gemm_run``, ``gemm_strided_run``, ``grouped_gemm_run``, ``mx_gemm_run``,
  ``mxfp4_gemm_run``, ``mxfp6_gemm_run``, ``mx_scales_blocks_bytes``,
  ``mx_scales_to_blocks``, ``mx_gemm_blocks_run``, ``gemm_layout_run``,
  ``gemm_layout128_run``, ``gemm_last_error``, ``gemm_version``,
  ``gemm_lds_layout``, ``gemm_lds_layout_mxfp6``, ``gemm_lds_layout_cblock``,
  ``gemm_lds_image``: the C entry points under the same names, taking integer
  device pointers.
* ``gemm``, ``gemm_strided``, ``grouped_gemm``, ``mx_gemm``, ``mxfp4_gemm``,
  ``mxfp6_gemm``, ``mx_scales_blocks``, ``mx_gemm_blocks``, ``gemm_layout``,
  ``gemm_layout128``: the same calls on torch CUDA
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
    "gemm_lds_image", "gemm_lds_image_tile", "gemm_mfma_scale_probe", "SG_IMG_HALF",
    "SG_IMG_HALF_KEXACT", "SG_IMG_MN256", "SG_IMG_FP6", "SG_IMG_CBLOCK", "gemm_last_kernel", "gemm_clock_trace", "gemm_clock_probe", "gemm_clock_probe_waves",
    "SG_E2M1", "SG_E2M3", "SG_E3M2", "SG_SF_ROWS", "SG_SF_BLOCKS",
    "mx_scales_blocks_bytes", "mx_scales_to_blocks", "mx_gemm_blocks_run", "mx_scales_blocks",
    "mx_gemm_blocks",
    "gemm", "gemm_plan", "gemm_strided", "grouped_gemm", "mx_gemm", "mxfp4_gemm", "mxfp6_gemm",
    "gemm_layout", "gemm_layout_io", "gemm_layout_io_run",
    "gemm_layout128", "SG_LAYOUT_PAD16",
    "library_path", "load",
]

SG_OK = 0
SG_NONE, SG_F16, SG_BF16, SG_F32, SG_E4M3, SG_E8M0 = 0, 1, 2, 3, 4, 5
SG_E2M1, SG_E2M3, SG_E3M2 = 6, 7, 8
SG_SF_ROWS, SG_SF_BLOCKS = 0, 1
SG_K_MAJOR, SG_MN_MAJOR = 0, 1
SG_MAX_GROUPS = 256
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
    lib.gemm_layout_io_run.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, i32, vp, i32, vp]
    lib.gemm_lds_layout.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_layout_mxfp6.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_layout_cblock.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_lds_image.argtypes = [vp, i64, i64, i32, i64, i64, i32, vp, vp]
    lib.gemm_lds_image_tile.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp]
    lib.gemm_mfma_scale_probe.argtypes = [i32, vp, vp, vp, vp, vp, vp]
    lib.gemm_clock_trace.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_int)]
    lib.gemm_clock_probe.argtypes = [i64, vp, vp]
    lib.gemm_clock_probe_waves.argtypes = []
    lib.mx_scales_blocks_bytes.argtypes = [i64, i64]
    lib.mx_scales_blocks_bytes.restype = ctypes.c_int64
    lib.mx_scales_to_blocks.argtypes = [vp, i64, i64, vp, vp]
    lib.mx_gemm_blocks_run.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp]
    for f in (lib.mx_scales_to_blocks, lib.mx_gemm_blocks_run, lib.gemm_run, lib.gemm_strided_run, lib.grouped_gemm_run, lib.mx_gemm_run,
              lib.mxfp4_gemm_run, lib.mxfp6_gemm_run,
              lib.gemm_layout_run, lib.gemm_layout128_run, lib.gemm_layout_io_run,
              lib.gemm_lds_layout, lib.gemm_lds_layout_mxfp6, lib.gemm_lds_layout_cblock,
              lib.gemm_lds_image, lib.gemm_lds_image_tile, lib.gemm_mfma_scale_probe,
              lib.gemm_clock_trace, lib.gemm_clock_probe,
              lib.gemm_clock_probe_waves):
        f.restype = ctypes.c_int
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_version.argtypes = []
    lib.gemm_version.restype = ctypes.c_char_p
    lib.gemm_last_kernel.argtypes = []
    lib.gemm_last_kernel.restype = ctypes.c_char_p
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


def mx_scales_blocks_bytes(rows, K) -> int:
    return load().mx_scales_blocks_bytes(rows, K)


def mx_scales_to_blocks(SF, rows, K, out, stream) -> int:
    return load().mx_scales_to_blocks(SF, rows, K, out, stream)


def mx_gemm_blocks_run(fmt, M, N, K, A, SFA, B, SFB, D, d_dtype, stream) -> int:
    return load().mx_gemm_blocks_run(fmt, M, N, K, A, SFA, B, SFB, D, d_dtype, stream)


def gemm_layout_run(swz_units, M, N, K, A, B, C, c_dtype, D, d_dtype, stream) -> int:
    return load().gemm_layout_run(swz_units, M, N, K, A, B, C, c_dtype, D, d_dtype, stream)


def gemm_layout_io_run(operand_swz, output_swz, M, N, K, A, B, C, c_dtype, D, d_dtype,
                       stream) -> int:
    return load().gemm_layout_io_run(operand_swz, output_swz, M, N, K, A, B, C, c_dtype, D,
                                     d_dtype, stream)


def gemm_layout128_run(layout, M, N, K, A, B, C, c_dtype, D, d_dtype, stream) -> int:
    return load().gemm_layout128_run(layout, M, N, K, A, B, C, c_dtype, D, d_dtype, stream)


def gemm_last_error() -> str:
    return load().gemm_last_error().decode()


def gemm_version() -> str:
    return load().gemm_version().decode()


def gemm_last_kernel() -> str:
    """The kernel instantiation the last launching call on this thread ran."""
    return load().gemm_last_kernel().decode()


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


SG_IMG_HALF, SG_IMG_HALF_KEXACT, SG_IMG_MN256, SG_IMG_FP6, SG_IMG_CBLOCK = 1, 2, 3, 4, 5


def gemm_lds_image_tile(kind, X, rows, row_bytes, row0, byte0, out, stream) -> int:
    return load().gemm_lds_image_tile(kind, X, rows, row_bytes, row0, byte0, out, stream)


def gemm_mfma_scale_probe(fmt, a, b, sa, sb, out, stream) -> int:
    return load().gemm_mfma_scale_probe(fmt, a, b, sa, sb, out, stream)


def gemm_clock_trace(buf, slots: int) -> int:
    """Turns the per-workgroup clock trace of later launches from this
    thread on (buf = device pointer of 4*slots uint64) or off (buf None);
    returns the real-time counter's rate in kHz."""
    khz = ctypes.c_int(0)
    _check(load().gemm_clock_trace(buf, int(slots), ctypes.byref(khz)))
    return khz.value


def gemm_clock_probe(iters: int, out, stream) -> int:
    return load().gemm_clock_probe(int(iters), out, stream)


def gemm_clock_probe_waves() -> int:
    return load().gemm_clock_probe_waves()


# ----------------------------------------------------------- torch convenience
#
# The wrappers check what the C ABI cannot see before they hand over any
# pointer: every tensor is 2-D (3-D for grouped B), densely packed (row-major,
# no transposed or expanded views) except where gemm_strided takes row
# strides, of the shape the problem implies, and on one CUDA device.  A
# failed check raises GemmError with the code of the matching C error:
# SG_ERR_SHAPE for shapes, SG_ERR_ALIGN for a layout the call cannot address,
# SG_ERR_DTYPE for element types, SG_ERR_NULL for a tensor that is not on the
# CUDA device of the others.  The device is checked last, so every other
# check also runs on CPU tensors.

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


def _need(cond: bool, code: int, msg: str) -> None:
    if not cond:
        raise GemmError(code, msg)


def _dense(name: str, t, dims: int = 2) -> None:
    """t is a packed row-major tensor of `dims` dimensions."""
    _need(t.dim() == dims, -3, f"{name} must be {dims}-D, got shape {tuple(t.shape)}")
    _need(t.is_contiguous(), -2,
          f"{name} must be contiguous (row-major, no transposed or expanded view); "
          f"strides {tuple(t.stride())}")


def _shape(name: str, t, shape) -> None:
    _need(tuple(t.shape) == tuple(shape), -3,
          f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_is(name: str, t, dtypes) -> None:
    _need(t.dtype in dtypes, -4, f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _one_device(*named) -> None:
    """Every (name, tensor) pair with a tensor lives on one CUDA device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        _need(t.device.type == "cuda", -1, f"{name} is on {t.device}, not a CUDA device")
        if dev is None:
            dev = t.device
        _need(t.device == dev, -1, f"{name} is on {t.device}, the others on {dev}")


def _mk(A, B, a_major: str, b_major: str):
    """(M, N, K) of A (a_major) and B (b_major), checking that K agrees."""
    _need(a_major in ("k", "mn") and b_major in ("k", "mn"), -5,
          f"majorness must be 'k' or 'mn', got {a_major!r}, {b_major!r}")
    M, K = A.shape if a_major == "k" else tuple(reversed(A.shape))
    N, Kb = B.shape if b_major == "k" else tuple(reversed(B.shape))
    _need(Kb == K, -3, f"A and B disagree on K ({K} vs {Kb})")
    _need(A.dtype == B.dtype, -4, f"A and B dtypes differ ({A.dtype} vs {B.dtype})")
    return int(M), int(N), int(K)


def _out(out, shape, dtype, device):
    """`out` checked against `shape`, or a new tensor of `dtype`."""
    import torch
    if out is None:
        return torch.empty(tuple(shape), dtype=dtype, device=device)
    _shape("out", out, shape)
    return out


def _gemm_args(A, B, a_major, b_major, C, out, out_dtype):
    """Checks of gemm()/gemm_plan(): returns (M, N, K, out)."""
    import torch
    _dense("A", A)
    _dense("B", B)
    M, N, K = _mk(A, B, a_major, b_major)
    _dtype_is("A", A, (torch.float16, torch.bfloat16))
    if C is not None:
        _dense("C", C)
        _shape("C", C, (M, N))
        _dtype_is("C", C, (torch.float32, torch.bfloat16, torch.float16))
    if out is not None:
        _dense("out", out)
        _shape("out", out, (M, N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16, torch.float16))
    _one_device(("A", A), ("B", B), ("C", C), ("out", out))
    out = _out(out, (M, N), out_dtype or torch.float32, A.device)
    return M, N, K, out


def gemm(A, B, *, a_major: str = "k", b_major: str = "k", C=None,
         out_dtype=None, out=None):
    """D = A*B (+C) on torch CUDA tensors.

    A: [M][K] (a_major "k") or [K][M] ("mn"); B: [N][K] ("k") or [K][N]
    ("mn"); C: optional [M][N]; returns D [M][N] of out_dtype (default
    torch.float32), or writes `out` [M][N].  Every tensor contiguous and on
    one CUDA device."""
    M, N, K, out = _gemm_args(A, B, a_major, b_major, C, out, out_dtype)
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
    otherwise take longer than the kernel.  The callable holds references to
    A, B, C and out, so their storage stays allocated while it lives; they
    must not be resized or have their storage replaced meanwhile."""
    _need(out is not None, -1, "gemm_plan needs out")
    M, N, K, out = _gemm_args(A, B, a_major, b_major, C, out, None)
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
    # The launch takes raw pointers: keep the tensors (and so their memory)
    # alive as long as the callable can be called.
    run.tensors = (A, B, C, out)
    return run


def _ld(t, name: str) -> int:
    _need(t.dim() == 2, -3, f"{name} must be 2-D, got shape {tuple(t.shape)}")
    _need(t.stride(1) == 1 and t.stride(0) >= max(t.shape[1], 1), -2,
          f"{name} must have unit column stride and a row stride of at least its width; "
          f"strides {tuple(t.stride())}")
    return t.stride(0)


def gemm_strided(A, B, *, a_major: str = "k", b_major: str = "k", C=None, alpha: float = 1.0,
                 beta: float = 1.0, out_dtype=None, out=None):
    """D = alpha * A*B + beta * C on 2-D torch CUDA tensors whose rows may be
    padded (views with unit column stride): leading dimensions are the row
    strides.  Shapes as in gemm(); `out` may itself be a padded view."""
    import torch
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    M, N, K = _mk(A, B, a_major, b_major)
    _dtype_is("A", A, (torch.float16, torch.bfloat16))
    if C is not None:
        ldc = _ld(C, "C")
        _shape("C", C, (M, N))
        _dtype_is("C", C, (torch.float32, torch.bfloat16, torch.float16))
    if out is not None:
        _shape("out", out, (M, N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16, torch.float16))
        ldd = _ld(out, "out")
    _one_device(("A", A), ("B", B), ("C", C), ("out", out))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=A.device)
        ldd = N
    _check(gemm_strided_run(M, N, K, float(alpha), A.data_ptr(), lda,
                            0 if a_major == "k" else 1, B.data_ptr(), ldb,
                            0 if b_major == "k" else 1, _dt(A.dtype), float(beta),
                            C.data_ptr() if C is not None else None,
                            ldc if C is not None else N,
                            _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                            ldd, _dt(out.dtype), _stream(A.device)))
    return out


def _layout_args(A, B, C, out, out_dtype):
    """Checks of the layout-ablation wrappers: bf16 K-major A [M][K] and
    B [N][K]."""
    import torch
    _dense("A", A)
    _dense("B", B)
    M, N, K = _mk(A, B, "k", "k")
    _dtype_is("A", A, (torch.bfloat16,))
    if C is not None:
        _dense("C", C)
        _shape("C", C, (M, N))
        _dtype_is("C", C, (torch.float32, torch.bfloat16, torch.float16))
    if out is not None:
        _dense("out", out)
        _shape("out", out, (M, N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16, torch.float16))
    _one_device(("A", A), ("B", B), ("C", C), ("out", out))
    return M, N, K, _out(out, (M, N), out_dtype or torch.float32, A.device)


def gemm_layout(A, B, swz_units: int, *, C=None, out_dtype=None, out=None):
    """gemm() for bf16 K-major A [M][K] and B [N][K] on the 256x256-tile
    kernel with the LDS layout swz_units (16 = the library's XOR swizzle
    over 256-byte lines, 8 = over 128-byte lines, 0 = none)."""
    M, N, K, out = _layout_args(A, B, C, out, out_dtype)
    _check(gemm_layout_run(swz_units, M, N, K, A.data_ptr(), B.data_ptr(),
                           C.data_ptr() if C is not None else None,
                           _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                           _dt(out.dtype), _stream(A.device)))
    return out


def gemm_layout_io(A, B, operand_swz: int, output_swz: int, *, C=None, out_dtype=None,
                   out=None):
    """gemm() for bf16 K-major A [M][K] and B [N][K] on the library's 256x256
    kernel with the operand layout operand_swz (16 or 0) and the epilogue's
    C/D staging swizzled (output_swz 1) or not (0); D is 16-bit (default
    bf16), C None or 16-bit."""
    import torch
    M, N, K, out = _layout_args(A, B, C, out, out_dtype or torch.bfloat16)
    _check(gemm_layout_io_run(operand_swz, output_swz, M, N, K, A.data_ptr(), B.data_ptr(),
                              C.data_ptr() if C is not None else None,
                              _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                              _dt(out.dtype), _stream(A.device)))
    return out


def gemm_layout128(A, B, layout: int, *, C=None, out_dtype=None, out=None):
    """gemm_layout() on 128x128 tiles, where layout may also be
    SG_LAYOUT_PAD16 (rows padded by 16 bytes, no swizzle)."""
    M, N, K, out = _layout_args(A, B, C, out, out_dtype)
    _check(gemm_layout128_run(layout, M, N, K, A.data_ptr(), B.data_ptr(),
                              C.data_ptr() if C is not None else None,
                              _dt(C.dtype) if C is not None else SG_NONE, out.data_ptr(),
                              _dt(out.dtype), _stream(A.device)))
    return out


def grouped_gemm(A, B, m_offsets: Sequence[int], *, out_dtype=None, out=None):
    """Per group g: D[off_g:off_{g+1}] = A[off_g:off_{g+1}] * B[g]^T.

    A: [sum M][K]; B: [G][N][K]; m_offsets: G+1 host ints (m_offsets[-1] is
    A's row count)."""
    import torch
    _dense("A", A)
    _dense("B", B, dims=3)
    G, N, K = (int(x) for x in B.shape)
    offs = [int(x) for x in m_offsets]
    _need(len(offs) == G + 1, -6, f"m_offsets has {len(offs)} entries, expected G+1 = {G + 1}")
    _need(A.shape[0] == offs[-1], -3,
          f"A has {A.shape[0]} rows, m_offsets[-1] = {offs[-1]}")
    _need(A.shape[1] == K, -3, f"A and B disagree on K ({A.shape[1]} vs {K})")
    _need(A.dtype == B.dtype, -4, f"A and B dtypes differ ({A.dtype} vs {B.dtype})")
    _dtype_is("A", A, (torch.float16, torch.bfloat16))
    if out is not None:
        _dense("out", out)
        _shape("out", out, (offs[-1], N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16, torch.float16))
    _one_device(("A", A), ("B", B), ("out", out))
    out = _out(out, (offs[-1], N), out_dtype or torch.bfloat16, A.device)
    _check(grouped_gemm_run(G, offs, N, K, A.data_ptr(), 0, B.data_ptr(), 0,
                            _dt(A.dtype), out.data_ptr(), _dt(out.dtype),
                            _stream(A.device)))
    return out


def _mx_args(A, SFA, B, SFB, out, out_dtype, k_per_byte_num: int, k_per_byte_den: int):
    """Checks of the block-scaled wrappers: uint8 A [M][bytes], B [N][bytes]
    with the same row bytes, SFA [M][K/32], SFB [N][K/32] uint8; returns
    (M, N, K, out)."""
    import torch
    for name, t in (("A", A), ("SFA", SFA), ("B", B), ("SFB", SFB)):
        _dense(name, t)
        _dtype_is(name, t, (torch.uint8,))
    M, N = int(A.shape[0]), int(B.shape[0])
    _need(A.shape[1] == B.shape[1], -3,
          f"A and B rows hold different byte counts ({A.shape[1]} vs {B.shape[1]})")
    K = int(A.shape[1]) * k_per_byte_num // k_per_byte_den
    _need(K * k_per_byte_den == int(A.shape[1]) * k_per_byte_num, -3,
          f"A's row of {A.shape[1]} bytes is not a whole number of elements")
    _shape("SFA", SFA, (M, K // 32))
    _shape("SFB", SFB, (N, K // 32))
    if out is not None:
        _dense("out", out)
        _shape("out", out, (M, N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16))
    _one_device(("A", A), ("SFA", SFA), ("B", B), ("SFB", SFB), ("out", out))
    return M, N, K, _out(out, (M, N), out_dtype or torch.bfloat16, A.device)


_MX_FMTS = {"e4m3": (SG_E4M3, 1, 1), "e2m1": (SG_E2M1, 2, 1), "e2m3": (SG_E2M3, 4, 3),
            "e3m2": (SG_E3M2, 4, 3)}


def mx_scales_blocks(SF, *, out=None):
    """e8m0 scales SF [rows][K/32] (uint8) rearranged into the SG_SF_BLOCKS
    layout: a 1-D uint8 tensor of mx_scales_blocks_bytes(rows, K) bytes
    (allocated by torch unless `out` is given)."""
    import torch
    _dense("SF", SF)
    _dtype_is("SF", SF, (torch.uint8,))
    rows, K = int(SF.shape[0]), int(SF.shape[1]) * 32
    n = int(mx_scales_blocks_bytes(rows, K))
    _check(n if n < 0 else 0)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=SF.device)
    else:
        _dense("out", out, 1)
        _shape("out", out, (n,))
        _dtype_is("out", out, (torch.uint8,))
    _one_device(("SF", SF), ("out", out))
    _check(mx_scales_to_blocks(SF.data_ptr(), rows, K, out.data_ptr(), _stream(SF.device)))
    return out


def mx_gemm_blocks(A, SFA, B, SFB, *, fmt: str = "e4m3", out_dtype=None, out=None):
    """The block-scaled GEMM of mx_gemm / mxfp4_gemm / mxfp6_gemm (fmt
    "e4m3", "e2m1", "e2m3" or "e3m2"; A and B as there) with SFA and SFB in
    the SG_SF_BLOCKS layout (mx_scales_blocks)."""
    import torch
    _need(fmt in _MX_FMTS, -4, f"fmt must be one of {sorted(_MX_FMTS)}, got {fmt!r}")
    code, num, den = _MX_FMTS[fmt]
    for name, t in (("A", A), ("B", B)):
        _dense(name, t)
        _dtype_is(name, t, (torch.uint8,))
    M, N = int(A.shape[0]), int(B.shape[0])
    _need(A.shape[1] == B.shape[1], -3,
          f"A and B rows hold different byte counts ({A.shape[1]} vs {B.shape[1]})")
    K = int(A.shape[1]) * num // den
    _need(K * den == int(A.shape[1]) * num, -3,
          f"A's row of {A.shape[1]} bytes is not a whole number of elements")
    for name, t, rows in (("SFA", SFA, M), ("SFB", SFB, N)):
        _dense(name, t, 1)
        _dtype_is(name, t, (torch.uint8,))
        n = int(mx_scales_blocks_bytes(rows, K))
        _check(n if n < 0 else 0)
        _shape(name, t, (n,))
    if out is not None:
        _dense("out", out)
        _shape("out", out, (M, N))
        _dtype_is("out", out, (torch.float32, torch.bfloat16))
    _one_device(("A", A), ("SFA", SFA), ("B", B), ("SFB", SFB), ("out", out))
    out = _out(out, (M, N), out_dtype or torch.bfloat16, A.device)
    _check(mx_gemm_blocks_run(code, M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                              SFB.data_ptr(), out.data_ptr(), _dt(out.dtype), _stream(A.device)))
    return out


def mx_gemm(A, SFA, B, SFB, *, out_dtype=None, out=None):
    """Block-scaled e4m3 GEMM: A [M][K], B [N][K] (uint8 e4m3 codes),
    SFA [M][K/32], SFB [N][K/32] (uint8 e8m0 codes)."""
    M, N, K, out = _mx_args(A, SFA, B, SFB, out, out_dtype, 1, 1)
    _check(mx_gemm_run(M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                       SFB.data_ptr(), out.data_ptr(), _dt(out.dtype),
                       _stream(A.device)))
    return out


def mxfp4_gemm(A, SFA, B, SFB, *, out_dtype=None, out=None):
    """Block-scaled e2m1 GEMM: A [M][K/2], B [N][K/2] (uint8, two e2m1 per
    byte, element 2i in the low nibble), SFA [M][K/32], SFB [N][K/32] (uint8
    e8m0 codes)."""
    M, N, K, out = _mx_args(A, SFA, B, SFB, out, out_dtype, 2, 1)
    _check(mxfp4_gemm_run(M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                          SFB.data_ptr(), out.data_ptr(), _dt(out.dtype), _stream(A.device)))
    return out


def mxfp6_gemm(A, SFA, B, SFB, *, fmt: str = "e2m3", out_dtype=None, out=None):
    """Block-scaled FP6 GEMM: A [M][3K/4], B [N][3K/4] (uint8, a 6-bit
    stream of e2m3 or e3m2 codes per row, element k at bits [6k, 6k+6)),
    SFA [M][K/32], SFB [N][K/32] (uint8 e8m0 codes)."""
    _need(fmt in ("e2m3", "e3m2"), -4, f"fmt must be 'e2m3' or 'e3m2', got {fmt!r}")
    code = {"e2m3": SG_E2M3, "e3m2": SG_E3M2}[fmt]
    M, N, K, out = _mx_args(A, SFA, B, SFB, out, out_dtype, 4, 3)
    _check(mxfp6_gemm_run(code, M, N, K, A.data_ptr(), SFA.data_ptr(), B.data_ptr(),
                          SFB.data_ptr(), out.data_ptr(), _dt(out.dtype), _stream(A.device)))
    return out
