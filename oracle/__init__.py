"""CPU oracle for the swizzled GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``dense_gemm_swizzled_amd``) and never imports it.

Contents
--------
* ``gemm`` / ``gemm_points``: fp64-accumulating triple loop of D = A*B (+C)
  over exactly decoded fp16/bf16 inputs, plus the per-element error bound
  ``sum_k |a*b| + |c|`` (``gemm_oracle.c``; the tensor-core operation of
  "Tensor Cores, layouts, and swizzling", opening section).
* ``gemm_ex``: the same sum read from strided storage, D = alpha*A*B +
  beta*C (leading dimensions as the tile copies of "Tensor Cores, layouts,
  and swizzling", Tensor Memory Accelerator section, address a tensor; the
  alpha/beta scaling is the plain reading of a scaled epilogue, the pages
  define none), with bound ``|alpha| sum_k |a*b| + |beta| |c|``.
* ``grouped_gemm``: the dense definition applied per group on rows
  ``[off_g, off_{g+1})`` with that group's B (the grouped GEMM named in
  "LBO, SBO and SWZ for a tcgen05 tile", introduction; the pages give no
  further definition, so this is the plain reading).
* ``mx_gemm`` / ``mx_gemm_points``: block-scaled GEMM with one e8m0 scale per
  row and 32-element K block ("06 Blackwell Tensor Core", Block-Scaled MMA);
  elements e4m3, e2m1 (two per byte) or e2m3 / e3m2 (a 6-bit stream).
* ``decode``: fp16 / bf16 / OCP e4m3, e2m1, e2m3, e3m2 / e8m0 decode to fp64.
* ``swizzle``: the XOR swizzle maps (``oracle.swizzle``).
* ``banks``: the LDS / shared-memory bank-conflict simulator
  (``oracle.banks``).

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, library routines on special cases and the pages'
worked examples.  No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_DT = {"f16": 1, "bf16": 2, "f32": 3, "e4m3": 4, "e8m0": 5, "e2m1": 6, "e2m3": 7,
       "e3m2": 8}
_MAJ = {"k": 0, "mn": 1}

_lib = None


def build(force: bool = True) -> str:
    """Compile gemm_oracle.c with gcc into liboracle.so (in-tree)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, dp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.oracle_decode.argtypes = [ip, vp, i64, dp]
        lib.oracle_gemm.argtypes = [i64, i64, i64, vp, ip, vp, ip, ip, vp, ip,
                                    dp, dp, ip]
        f64 = ctypes.c_double
        lib.oracle_gemm_ex.argtypes = [i64, i64, i64, f64, vp, i64, ip, vp, i64, ip, ip,
                                       f64, vp, i64, ip, dp, dp, ip]
        lib.oracle_gemm_points.argtypes = [i64, i64, i64, vp, ip, vp, ip, ip,
                                           vp, ip, i64, vp, vp, dp, dp]
        lib.oracle_mx_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, dp, dp, ip]
        lib.oracle_mx_gemm_points.argtypes = [i64, i64, i64, vp, vp, vp, vp,
                                              i64, vp, vp, dp, dp]
        lib.oracle_mx_gemm_fmt.argtypes = [ip, i64, i64, i64, vp, vp, vp, vp, dp, dp, ip]
        lib.oracle_mx_gemm_points_fmt.argtypes = [ip, i64, i64, i64, vp, vp, vp, vp,
                                                  i64, vp, vp, dp, dp]
        lib.oracle_default_threads.argtypes = []
        for f in (lib.oracle_decode, lib.oracle_gemm, lib.oracle_gemm_ex, lib.oracle_gemm_points,
                  lib.oracle_mx_gemm, lib.oracle_mx_gemm_points,
                  lib.oracle_mx_gemm_fmt, lib.oracle_mx_gemm_points_fmt,
                  lib.oracle_default_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return _load().oracle_default_threads()


def _bytes(x) -> np.ndarray:
    """CPU tensor / ndarray -> contiguous numpy array sharing its bytes."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU)
        import torch
        t = x.detach().contiguous()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be CPU tensors")
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.view(torch.int16).numpy()
        if t.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
            return t.view(torch.uint8).numpy()
        return t.numpy()
    return np.ascontiguousarray(x)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(dtype: str, data) -> np.ndarray:
    """Decode raw storage of ``dtype`` ("f16", "bf16", "f32", "e4m3",
    "e8m0", "e2m1", "e2m3", "e3m2") to fp64, element by element.  e2m1 packs
    two elements per byte (element 2i in the low nibble of byte i) and
    returns a flat array of 2 * nbytes values; e2m3 and e3m2 are a 6-bit
    stream (element k at bits [6k, 6k+6), little endian) and return
    nbytes * 4 / 3 values."""
    a = _bytes(data)
    if dtype in ("e2m1", "e2m3", "e3m2"):
        n = a.nbytes * 2 if dtype == "e2m1" else a.nbytes * 4 // 3
        out = np.empty(n, dtype=np.float64)
        if _load().oracle_decode(_DT[dtype], _ptr(a), n, _ptr(out)) != 0:
            raise ValueError("oracle_decode failed")
        return out
    width = {"f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e8m0": 1}[dtype]
    n = a.nbytes // width
    out = np.empty(n, dtype=np.float64)
    if _load().oracle_decode(_DT[dtype], _ptr(a), n, _ptr(out)) != 0:
        raise ValueError("oracle_decode failed")
    return out.reshape(a.shape) if a.itemsize == width else out


def gemm(M: int, N: int, K: int, A, a_major: str, B, b_major: str,
         ab_dtype: str, C=None, c_dtype: Optional[str] = None,
         nthreads: int = 0, with_bound: bool = True):
    """ref, bound = fp64 D = A*B (+C) and sum|a*b| (+|c|), both [M][N]."""
    a, b, c = _bytes(A), _bytes(B), _bytes(C)
    ref = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_gemm(M, N, K, _ptr(a), _MAJ[a_major], _ptr(b),
                             _MAJ[b_major], _DT[ab_dtype], _ptr(c),
                             _DT[c_dtype] if c is not None else 0,
                             _ptr(ref), _ptr(bound), nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return ref, bound


def gemm_ex(M: int, N: int, K: int, alpha: float, A, lda: int, a_major: str, B, ldb: int,
            b_major: str, ab_dtype: str, beta: float, C=None, ldc: int = 0,
            c_dtype: Optional[str] = None, nthreads: int = 0, with_bound: bool = True):
    """ref, bound = fp64 D = alpha*A*B + beta*C and |alpha|sum|a*b| + |beta||c|
    from strided storage (leading dimensions in elements; A, B, C are the
    whole buffers).  alpha == 0 reads neither A nor B; beta == 0 does not
    read C."""
    a, b, c = _bytes(A), _bytes(B), _bytes(C)
    ref = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_gemm_ex(M, N, K, float(alpha), _ptr(a), lda, _MAJ[a_major],
                                _ptr(b), ldb, _MAJ[b_major], _DT[ab_dtype],
                                float(beta), _ptr(c), ldc,
                                _DT[c_dtype] if c is not None else 0,
                                _ptr(ref), _ptr(bound), nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm_ex rejected its arguments")
    return ref, bound


def gemm_points(M: int, N: int, K: int, A, a_major: str, B, b_major: str,
                ab_dtype: str, rows: Sequence[int], cols: Sequence[int],
                C=None, c_dtype: Optional[str] = None):
    """The dense definition at the listed (row, col) points only."""
    a, b, c = _bytes(A), _bytes(B), _bytes(C)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    q = np.ascontiguousarray(cols, dtype=np.int64)
    ref = np.empty(len(r), dtype=np.float64)
    bound = np.empty(len(r), dtype=np.float64)
    rc = _load().oracle_gemm_points(M, N, K, _ptr(a), _MAJ[a_major], _ptr(b),
                                    _MAJ[b_major], _DT[ab_dtype], _ptr(c),
                                    _DT[c_dtype] if c is not None else 0,
                                    len(r), _ptr(r), _ptr(q), _ptr(ref),
                                    _ptr(bound))
    if rc != 0:
        raise ValueError("oracle_gemm_points rejected its arguments")
    return ref, bound


def grouped_gemm(m_offsets: Sequence[int], N: int, K: int, A, B,
                 ab_dtype: str, nthreads: int = 0):
    """Per group g: rows [off_g, off_{g+1}) of D = those rows of A times B_g.

    A is K-major [sum M][K]; B is K-major [G][N][K].  Returns fp64 ref and
    bound of shape [sum M][N]."""
    a, b = _bytes(A), _bytes(B)
    G = len(m_offsets) - 1
    total = int(m_offsets[-1])
    ref = np.empty((total, N), dtype=np.float64)
    bound = np.empty((total, N), dtype=np.float64)
    a2 = a.reshape(total, K) if total else a
    b3 = b.reshape(G, N, K)
    for g in range(G):
        lo, hi = int(m_offsets[g]), int(m_offsets[g + 1])
        if hi <= lo:
            continue
        r, bd = gemm(hi - lo, N, K, np.ascontiguousarray(a2[lo:hi]), "k",
                     np.ascontiguousarray(b3[g]), "k", ab_dtype,
                     nthreads=nthreads)
        ref[lo:hi] = r
        bound[lo:hi] = bd
    return ref, bound


def mx_gemm(M: int, N: int, K: int, A, SFA, B, SFB, nthreads: int = 0,
            with_bound: bool = True, fmt: str = "e4m3"):
    """Block-scaled GEMM with e8m0 scales per 32-element K block; the
    elements are e4m3 (A [M][K] bytes), e2m1 (fmt "e2m1", A [M][K/2]
    bytes, two elements per byte) or e2m3 / e3m2 (A [M][3K/4] bytes, a
    6-bit stream per row)."""
    a, sa, b, sb = _bytes(A), _bytes(SFA), _bytes(B), _bytes(SFB)
    ref = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = _load().oracle_mx_gemm_fmt(_DT[fmt], M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                    _ptr(ref), _ptr(bound), nthreads)
    if rc != 0:
        raise ValueError("oracle_mx_gemm rejected its arguments")
    return ref, bound


def mx_gemm_points(M: int, N: int, K: int, A, SFA, B, SFB,
                   rows: Sequence[int], cols: Sequence[int], fmt: str = "e4m3"):
    a, sa, b, sb = _bytes(A), _bytes(SFA), _bytes(B), _bytes(SFB)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    q = np.ascontiguousarray(cols, dtype=np.int64)
    ref = np.empty(len(r), dtype=np.float64)
    bound = np.empty(len(r), dtype=np.float64)
    rc = _load().oracle_mx_gemm_points_fmt(_DT[fmt], M, N, K, _ptr(a), _ptr(sa), _ptr(b),
                                           _ptr(sb), len(r), _ptr(r), _ptr(q),
                                           _ptr(ref), _ptr(bound))
    if rc != 0:
        raise ValueError("oracle_mx_gemm_points rejected its arguments")
    return ref, bound


from . import swizzle, banks  # noqa: E402,F401
