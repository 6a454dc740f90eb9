"""Seeded synthetic inputs for the swizzled GEMM workloads.

This module only draws random numbers and rounds them to the storage formats
the GEMM consumes (fp16, bf16, and the OCP MX element formats e4m3, e2m1,
e2m3 and e3m2 with e8m0 block scales).  It holds
none of the GEMM arithmetic: the same bytes it returns are handed to the CPU
oracle and to the HIP path, and each side computes from them on its own.

Every generator takes an explicit seed and draws in a fixed order from
``numpy.random.default_rng(seed)`` (PCG64).  Draws are fp32 and are rounded
to the 16-bit types with torch CPU casts (round-to-nearest-even).

Workloads (sizes, majorness and distributions of the five GEMM cases):

* ``single_tile``: M=128, N=128, K=32 fp16, A K-major ``[M][K]``, B MN-major
  ``[K][N]``, entries U[-1,1].
* ``dense_1024``: M=N=K=1024 bf16, A K-major, B MN-major ``[K][N]``,
  entries N(0,1), no C.
* ``dense_8192``: M=N=K=8192 bf16, A and B K-major (B stored ``[N][K]``),
  entries N(0,1)/sqrt(K); C ~ N(0,1) bf16 is added; bf16 output.
* ``grouped``: 16 groups, N=K=4096 bf16, per-group M_i = 128*U{1..16};
  A ``[sum M_i][K]`` K-major, B ``[G][N][K]`` K-major, entries N(0,1)/sqrt(K).
* ``mxfp8``: M=N=K=8192, A ``[M][K]``, B ``[N][K]``, N(0,1) fp32 values
  quantised per 32-element K block to e4m3 with an e8m0 scale equal to the
  power of two at or below the block's absolute maximum.
* ``mxfp4``: the same shape with e2m1 elements (two per byte), the scale
  putting each block's absolute maximum in e2m1's top binade [4, 8).
* ``mxfp6``: the same shape with e2m3 (or e3m2) elements in a 6-bit stream,
  the scale putting each block's absolute maximum in the format's top
  binade ([4, 8) for e2m3, [16, 32) for e3m2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Operand", "DenseCase", "GroupedCase", "MXCase",
    "uniform", "normal", "to_fp16", "to_bf16", "mx_quantize",
    "single_tile", "dense_1024", "dense_8192", "grouped", "mxfp8", "mxfp4",
    "mxfp4_quantize",
    "dense_case", "grouped_case", "mx_case", "integer_valued",
]

K_MAJOR = "k"
MN_MAJOR = "mn"


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform(rng: np.random.Generator, shape, lo=-1.0, hi=1.0) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def normal(rng: np.random.Generator, shape, scale=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_fp16(x: np.ndarray) -> torch.Tensor:
    """fp32 -> fp16 (round to nearest even), CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float16)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 -> bf16 (round to nearest even), CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f16":
        return to_fp16(x)
    if dtype == "bf16":
        return to_bf16(x)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.float32)))
    raise ValueError(dtype)


@dataclass
class DenseCase:
    """Storage of one dense problem; tensors are CPU and contiguous."""
    M: int
    N: int
    K: int
    A: torch.Tensor          # [M][K] if a_major == "k" else [K][M]
    a_major: str
    B: torch.Tensor          # [N][K] if b_major == "k" else [K][N]
    b_major: str
    ab_dtype: str            # "f16" | "bf16"
    C: Optional[torch.Tensor]  # [M][N] or None
    c_dtype: Optional[str]
    d_dtype: str             # "f32" | "bf16"
    name: str = ""


@dataclass
class GroupedCase:
    G: int
    m_sizes: list
    m_offsets: list          # G+1 prefix sums, offsets[0] = 0
    N: int
    K: int
    A: torch.Tensor          # [sum M][K] K-major
    B: torch.Tensor          # [G][N][K] K-major
    ab_dtype: str
    d_dtype: str
    name: str = ""


@dataclass
class MXCase:
    M: int
    N: int
    K: int
    A: torch.Tensor          # uint8 e4m3 [M][K], e2m1 [M][K/2] or fp6 [M][3K/4]
    SFA: torch.Tensor        # uint8 e8m0 [M][K/32]
    B: torch.Tensor          # uint8 e4m3 [N][K], e2m1 [N][K/2] or fp6 [N][3K/4]
    SFB: torch.Tensor        # uint8 e8m0 [N][K/32]
    d_dtype: str
    name: str = ""
    fmt: str = "e4m3"        # element format: "e4m3", "e2m1", "e2m3" or "e3m2"


def _layout(x_logical: np.ndarray, major: str) -> np.ndarray:
    """x_logical is [rows][K]; K-major keeps it, MN-major stores [K][rows]."""
    return x_logical if major == K_MAJOR else np.ascontiguousarray(x_logical.T)


def dense_case(M, N, K, seed, *, ab_dtype="bf16", a_major=K_MAJOR,
               b_major=K_MAJOR, dist="normal", scale=1.0, with_c=False,
               c_dtype="bf16", d_dtype="f32", name="") -> DenseCase:
    """Generic dense problem.  Draw order: A (logical [M][K] row-major),
    then B (logical [N][K] if K-major else [K][N]), then C."""
    rng = _rng(seed)
    draw = (lambda s: uniform(rng, s)) if dist == "uniform" else \
           (lambda s: normal(rng, s, scale))
    a = draw((M, K))
    if b_major == K_MAJOR:
        b = draw((N, K))
    else:
        b = draw((K, N))
    c = normal(rng, (M, N)) if with_c else None
    A = to_dtype(_layout(a, a_major), ab_dtype)
    B = to_dtype(b, ab_dtype)
    C = to_dtype(c, c_dtype) if with_c else None
    return DenseCase(M, N, K, A, a_major, B, b_major, ab_dtype, C,
                     c_dtype if with_c else None, d_dtype, name)


def single_tile(seed: int = 1) -> DenseCase:
    """128x128x32 fp16, A K-major, B MN-major [K][N], U[-1,1], fp32 out."""
    return dense_case(128, 128, 32, seed, ab_dtype="f16", a_major=K_MAJOR,
                      b_major=MN_MAJOR, dist="uniform", d_dtype="f32",
                      name="single_tile_128x128x32_f16")


def dense_1024(seed: int = 2) -> DenseCase:
    """1024^3 bf16, A K-major, B [K][N], N(0,1), fp32 out, no C."""
    return dense_case(1024, 1024, 1024, seed, ab_dtype="bf16",
                      a_major=K_MAJOR, b_major=MN_MAJOR, dist="normal",
                      d_dtype="f32", name="dense_1024_bf16")


def dense_8192(seed: int = 3, M: int = 8192, N: int = 8192,
               K: int = 8192) -> DenseCase:
    """8192^3 bf16, A and B K-major, N(0,1)/sqrt(K), + C~N(0,1) bf16, bf16 out."""
    return dense_case(M, N, K, seed, ab_dtype="bf16", a_major=K_MAJOR,
                      b_major=K_MAJOR, dist="normal", scale=1.0 / math.sqrt(K),
                      with_c=True, c_dtype="bf16", d_dtype="bf16",
                      name=f"dense_{M}x{N}x{K}_bf16_c")


def grouped_case(m_sizes, N, K, seed, *, ab_dtype="bf16", d_dtype="bf16",
                 name="") -> GroupedCase:
    rng = _rng(seed)
    m_sizes = [int(m) for m in m_sizes]
    offs = [0]
    for m in m_sizes:
        offs.append(offs[-1] + m)
    scale = 1.0 / math.sqrt(K)
    a = normal(rng, (offs[-1], K), scale)
    b = normal(rng, (len(m_sizes), N, K), scale)
    return GroupedCase(len(m_sizes), m_sizes, offs, N, K,
                       to_dtype(a, ab_dtype), to_dtype(b, ab_dtype),
                       ab_dtype, d_dtype, name)


def grouped(seed: int = 4, G: int = 16, N: int = 4096, K: int = 4096,
            m_unit: int = 128, m_max_units: int = 16) -> GroupedCase:
    """16 groups, M_i = 128 * U{1..16} from the seed, N=K=4096 bf16."""
    rng = _rng(seed)
    m_sizes = (m_unit * rng.integers(1, m_max_units + 1, G)).tolist()
    # A and B draws continue from a second stream keyed on the same seed so
    # that the sizes alone can be reproduced cheaply.
    return grouped_case(m_sizes, N, K, seed + 1000,
                        name=f"grouped_{G}x{N}x{K}_bf16")


def mx_quantize(x: np.ndarray, block: int = 32):
    """Quantise fp32 rows [R][K] to e4m3 with one e8m0 scale per K block.

    The scale is X = 2^floor(log2(absmax)) of the block (X = 1 for an
    all-zero block); elements are e4m3(x / X), rounded to nearest even by
    torch's float8_e4m3fn cast.  Since |x/X| < 2 no element saturates.
    Returns (codes uint8 [R][K], scales uint8 [R][K/block]).
    """
    R, K = x.shape
    assert K % block == 0
    xb = x.reshape(R, K // block, block)
    amax = np.abs(xb).max(axis=2)
    e = np.zeros_like(amax, dtype=np.int32)
    nz = amax > 0
    # frexp gives amax = f * 2^ex with f in [0.5, 1): floor(log2) = ex - 1.
    _, ex = np.frexp(amax[nz])
    e[nz] = ex - 1
    xs = xb / np.ldexp(np.float32(1.0), e)[:, :, None].astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(xs.reshape(R, K))).to(
        torch.float8_e4m3fn).view(torch.uint8)
    scales = torch.from_numpy((e + 127).astype(np.uint8))
    return codes, scales


# e2m1 magnitudes by code, and the rounding thresholds between neighbours:
# a tie goes to the even code (fraction bit 0).
_E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
_E2M1_MIDS = (_E2M1_VALUES[:-1] + _E2M1_VALUES[1:]) / 2


def mxfp4_quantize(x: np.ndarray, block: int = 32):
    """Quantise fp32 rows [R][K] to e2m1 with one e8m0 scale per K block.

    The scale is X = 2^(floor(log2(absmax)) - 2) of the block (X = 1 for an
    all-zero block), which puts the block's largest magnitude in [4, 8), the
    top binade of e2m1 (largest value 6; larger magnitudes become 6).
    Elements are x / X rounded to the nearest e2m1 value, ties to the even
    code.  Two elements per byte, element 2i in the low nibble of byte i.
    Returns (packed uint8 [R][K/2], scales uint8 [R][K/block]).
    """
    R, K = x.shape
    assert K % block == 0 and K % 2 == 0
    xb = x.reshape(R, K // block, block)
    amax = np.abs(xb).max(axis=2)
    e = np.zeros_like(amax, dtype=np.int32)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    e[nz] = ex - 1 - 2
    e = np.clip(e, -127, 127)
    y = (xb / np.ldexp(np.float32(1.0), e)[:, :, None].astype(np.float32)).reshape(R, K)
    mag = np.minimum(np.abs(y), np.float32(6.0))
    code = np.zeros(mag.shape, dtype=np.uint8)
    for i, t in enumerate(_E2M1_MIDS):
        # between codes i and i+1: a tie rounds to the even one
        code += (mag >= t) if i % 2 else (mag > t)
    code |= ((y < 0) & (code != 0)).astype(np.uint8) << 3
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(np.ascontiguousarray(packed)), torch.from_numpy((e + 127).astype(np.uint8))


def _fp6_magnitudes(exp_bits: int, man_bits: int) -> np.ndarray:
    """Magnitudes of the 32 non-negative codes of an OCP FP6 format with
    1 + exp_bits + man_bits = 6 bits and no Inf/NaN (E2M3: bias 1, E3M2:
    bias 3); code c has exponent field c >> man_bits, fraction c & mask."""
    bias = (1 << (exp_bits - 1)) - 1
    out = np.empty(32, dtype=np.float64)
    for c in range(32):
        e, m = c >> man_bits, c & ((1 << man_bits) - 1)
        if e == 0:
            out[c] = math.ldexp(m, 1 - bias - man_bits)
        else:
            out[c] = math.ldexp((1 << man_bits) + m, e - bias - man_bits)
    return out


# name -> (exponent bits, fraction bits, exponent of the top binade)
_FP6 = {"e2m3": (2, 3, 2), "e3m2": (3, 2, 4)}


def mxfp6_quantize(x: np.ndarray, fmt: str = "e2m3", block: int = 32):
    """Quantise fp32 rows [R][K] to FP6 (``fmt`` "e2m3" or "e3m2") with one
    e8m0 scale per K block.

    The scale is X = 2^(floor(log2(absmax)) - emax) of the block (emax = 2
    for E2M3, 4 for E3M2; X = 1 for an all-zero block), which puts the
    block's largest magnitude in the format's top binade; magnitudes above
    the largest value (7.5 resp. 28) become it.  Elements are x / X rounded
    to the nearest value, ties to the even code.  The codes of a row form a
    6-bit stream: element k at bits [6k, 6k + 6), little endian, so four
    elements fill three bytes.
    Returns (packed uint8 [R][3K/4], scales uint8 [R][K/block]).
    """
    eb, mb, emax = _FP6[fmt]
    R, K = x.shape
    assert K % block == 0 and K % 4 == 0
    xb = x.reshape(R, K // block, block)
    amax = np.abs(xb).max(axis=2)
    e = np.zeros_like(amax, dtype=np.int32)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    e[nz] = ex - 1 - emax
    e = np.clip(e, -127, 127)
    y = (xb / np.ldexp(np.float32(1.0), e)[:, :, None].astype(np.float32)).reshape(R, K)
    vals = _fp6_magnitudes(eb, mb).astype(np.float32)
    mids = (vals[:-1] + vals[1:]) / 2
    mag = np.minimum(np.abs(y), vals[-1])
    # below = number of midpoints under mag; a tie between codes i and i+1
    # (mag == mids[i], i = below) goes to the even one
    below = np.searchsorted(mids, mag, side="left").astype(np.uint32)
    tie = mag == mids[np.minimum(below, len(mids) - 1)]
    code = below + (tie & (below % 2 == 1)).astype(np.uint32)
    code |= ((y < 0) & (code != 0)).astype(np.uint32) << 5
    q = code.reshape(R, K // 4, 4)
    w = q[:, :, 0] | (q[:, :, 1] << 6) | (q[:, :, 2] << 12) | (q[:, :, 3] << 18)
    packed = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=2).astype(np.uint8)
    return (torch.from_numpy(np.ascontiguousarray(packed.reshape(R, 3 * K // 4))),
            torch.from_numpy((e + 127).astype(np.uint8)))


def mx_case(M, N, K, seed, *, d_dtype="bf16", name="", fmt="e4m3") -> MXCase:
    rng = _rng(seed)
    a = normal(rng, (M, K))
    b = normal(rng, (N, K))
    if fmt == "e4m3":
        q = mx_quantize
    elif fmt == "e2m1":
        q = mxfp4_quantize
    else:
        q = lambda v: mxfp6_quantize(v, fmt)  # noqa: E731
    A, SFA = q(a)
    B, SFB = q(b)
    return MXCase(M, N, K, A, SFA, B, SFB, d_dtype, name, fmt)


def mxfp8(seed: int = 5, M: int = 8192, N: int = 8192, K: int = 8192) -> MXCase:
    """MXFP8 8192^3: e4m3 with per-32 K-block e8m0 scales, bf16 out."""
    return mx_case(M, N, K, seed, name=f"mxfp8_{M}x{N}x{K}")


def mxfp4(seed: int = 7, M: int = 8192, N: int = 8192, K: int = 8192) -> MXCase:
    """MXFP4 8192^3: e2m1 (two per byte) with per-32 K-block e8m0 scales, bf16 out."""
    return mx_case(M, N, K, seed, name=f"mxfp4_{M}x{N}x{K}", fmt="e2m1")


def mxfp6(seed: int = 8, M: int = 8192, N: int = 8192, K: int = 8192,
          fmt: str = "e2m3") -> MXCase:
    """MXFP6 8192^3: e2m3 (or e3m2) as a 6-bit stream with per-32 K-block
    e8m0 scales, bf16 out."""
    return mx_case(M, N, K, seed, name=f"mxfp6_{fmt}_{M}x{N}x{K}", fmt=fmt)


def integer_valued(shape, seed, lo=-4, hi=4) -> np.ndarray:
    """Integer-valued fp32 draws in [lo, hi] (exact in fp16/bf16/e4m3)."""
    rng = _rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)
