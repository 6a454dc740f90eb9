"""Pins of the oracle's block-scaled (MX) and grouped GEMMs (CPU only).

MX: the e4m3 / e8m0 decode is checked on all 256 codes against torch's
float8_e4m3fn / float8_e8m0fnu conversions and against closed-form values;
the e2m1 (MXFP4) decode against the format's documented value set, its
nibble order and exact representability in e4m3 (torch's cast);
the GEMM against numpy on special cases (unit scales = plain fp8 GEMM, a
single rescaled block, integer values with power-of-two scales).
Grouped: G = 1 equals the dense GEMM; the result is the concatenation of
per-group numpy products; empty groups produce no rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si


def test_e4m3_all_codes_match_torch_and_closed_forms():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ours = oracle.decode("e4m3", codes)
    theirs = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], theirs[~nan])
    # Closed forms of OCP E4M3 (bias 7, 3 fraction bits, max 448).
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0
    assert ours[0x7E] == 448.0
    assert ours[0x08] == 2.0 ** -6          # smallest normal
    assert ours[0x01] == 2.0 ** -9          # smallest subnormal
    assert ours[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert ours[0x00] == 0.0 and ours[0x80] == 0.0


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ours = oracle.decode("e8m0", codes)
    assert np.isnan(ours[255])
    assert np.array_equal(ours[:255], np.ldexp(1.0, np.arange(255) - 127))
    theirs = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ours[:255], theirs[:255])


def _fp8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x.astype(np.float32))).to(
        torch.float8_e4m3fn).view(torch.uint8)


def _dec8(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_unit_scales_equal_plain_fp8_gemm():
    M, N, K = 7, 9, 96
    rng = np.random.default_rng(1)
    A = _fp8(rng.standard_normal((M, K)))
    B = _fp8(rng.standard_normal((N, K)))
    SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ref, bound = oracle.mx_gemm(M, N, K, A, SFA, B, SFB)
    expect = _dec8(A) @ _dec8(B).T
    assert np.allclose(ref, expect, rtol=1e-14, atol=1e-14)
    assert np.allclose(bound, np.abs(_dec8(A)) @ np.abs(_dec8(B)).T, rtol=1e-14)


def test_each_scale_applies_to_its_own_row_column_and_block():
    M, N, K = 4, 3, 128
    rng = np.random.default_rng(2)
    a = si.integer_valued((M, K), 3, -3, 3)
    b = si.integer_valued((N, K), 4, -3, 3)
    A, B = _fp8(a), _fp8(b)
    sa = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    ref, _ = oracle.mx_gemm(M, N, K, A, torch.from_numpy(sa), B, torch.from_numpy(sb))
    # Integer values times powers of two: every term and sum is exact.
    expect = np.zeros((M, N))
    for blk in range(K // 32):
        sl = slice(32 * blk, 32 * blk + 32)
        part = a[:, sl].astype(np.float64) @ b[:, sl].astype(np.float64).T
        expect += part * np.ldexp(1.0, sa[:, blk].astype(np.int64) - 127)[:, None] \
                       * np.ldexp(1.0, sb[:, blk].astype(np.int64) - 127)[None, :]
    assert np.array_equal(ref, expect)
    # Raising only SFA[1][2] by 3 changes only row 1, by 7x block 2's share.
    sa2 = sa.copy()
    sa2[1, 2] += 3
    ref2, _ = oracle.mx_gemm(M, N, K, A, torch.from_numpy(sa2), B, torch.from_numpy(sb))
    blk2 = (a[1, 64:96].astype(np.float64) @ b[:, 64:96].astype(np.float64).T) \
        * 2.0 ** (int(sa[1, 2]) - 127) * np.ldexp(1.0, sb[:, 2].astype(np.int64) - 127)
    assert np.array_equal(np.delete(ref2, 1, 0), np.delete(ref, 1, 0))
    assert np.array_equal(ref2[1], ref[1] + 7 * blk2)


def test_mx_points_agree_with_full():
    case = si.mx_case(40, 24, 160, 9)
    ref, bound = oracle.mx_gemm(case.M, case.N, case.K, case.A, case.SFA, case.B, case.SFB)
    rows, cols = [0, 39, 17], [0, 23, 5]
    rp, bp = oracle.mx_gemm_points(case.M, case.N, case.K, case.A, case.SFA,
                                   case.B, case.SFB, rows, cols)
    assert np.array_equal(rp, ref[rows, cols]) and np.array_equal(bp, bound[rows, cols])


def test_mx_quantizer_scale_is_power_of_two_at_or_below_absmax():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[2, 32:64] = 0.0
    codes, scales = si.mx_quantize(x)
    xb = x.reshape(6, 8, 32)
    amax = np.abs(xb).max(axis=2)
    X = np.ldexp(1.0, scales.numpy().astype(np.int64) - 127)
    nz = amax > 0
    assert np.all(X[nz] <= amax[nz]) and np.all(amax[nz] < 2 * X[nz])
    assert X[2, 1] == 1.0
    dec = _dec8(codes).reshape(6, 8, 32)
    assert np.all(np.abs(dec) <= 2.0)  # |x/X| < 2 may round up to 2
    # Dequantised values are within half an e4m3 step (2^-3 relative) of x.
    deq = dec * X[:, :, None]
    assert np.all(np.abs(deq - xb) <= 2.0 ** -4 * X[:, :, None] + 1e-30)


# ------------------------------------------------------------------ MXFP4

# The OCP FP4 E2M1 value set: positive codes 0..7 in order, negative codes
# 8..15 their mirror.  Written as a literal list, not from the encoding.
E2M1_DOCUMENTED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _unpack4(packed: torch.Tensor) -> np.ndarray:
    """numpy decode of packed e2m1 through the documented value list."""
    p = packed.numpy().astype(np.int64)
    lo, hi = p & 15, p >> 4
    table = np.array(E2M1_DOCUMENTED + [-v for v in E2M1_DOCUMENTED])
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],))
    out[..., 0::2] = table[lo]
    out[..., 1::2] = table[hi]
    return out


def test_e2m1_all_codes_match_documented_values():
    codes = np.arange(16, dtype=np.uint8)
    ours = oracle.decode("e2m1", codes | (codes << 4))   # byte c holds c twice
    assert np.array_equal(ours[0::2], ours[1::2])
    vals = ours[0::2]
    assert vals[:8].tolist() == E2M1_DOCUMENTED
    assert vals[8:].tolist() == [-v for v in E2M1_DOCUMENTED]
    # every value is exactly an e4m3 value (torch's cast is a library routine)
    t = torch.tensor(vals).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(t, vals)
    # element 2i is the low nibble of byte i
    assert oracle.decode("e2m1", np.array([0x71], dtype=np.uint8)).tolist() == [0.5, 6.0]


def test_e2m1_unit_scales_equal_plain_fp4_gemm():
    M, N, K = 6, 5, 128
    rng = np.random.default_rng(11)
    A = torch.from_numpy(rng.integers(0, 256, (M, K // 2)).astype(np.uint8))
    B = torch.from_numpy(rng.integers(0, 256, (N, K // 2)).astype(np.uint8))
    SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ref, bound = oracle.mx_gemm(M, N, K, A, SFA, B, SFB, fmt="e2m1")
    a, b = _unpack4(A), _unpack4(B)
    # e2m1 values are multiples of 1/2 below 8: every product and sum is exact
    assert np.array_equal(ref, a @ b.T)
    assert np.array_equal(bound, np.abs(a) @ np.abs(b).T)


def test_e2m1_each_scale_applies_to_its_own_block():
    M, N, K = 3, 4, 96
    rng = np.random.default_rng(12)
    A = torch.from_numpy(rng.integers(0, 256, (M, K // 2)).astype(np.uint8))
    B = torch.from_numpy(rng.integers(0, 256, (N, K // 2)).astype(np.uint8))
    sa = rng.integers(118, 137, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    ref, _ = oracle.mx_gemm(M, N, K, A, torch.from_numpy(sa), B, torch.from_numpy(sb),
                            fmt="e2m1")
    a, b = _unpack4(A), _unpack4(B)
    expect = np.zeros((M, N))
    for blk in range(K // 32):
        sl = slice(32 * blk, 32 * blk + 32)
        expect += (a[:, sl] @ b[:, sl].T) * np.ldexp(1.0, sa[:, blk].astype(np.int64) - 127)[:, None] \
            * np.ldexp(1.0, sb[:, blk].astype(np.int64) - 127)[None, :]
    assert np.array_equal(ref, expect)


def test_e2m1_points_agree_with_full():
    case = si.mx_case(33, 20, 256, 13, fmt="e2m1")
    ref, bound = oracle.mx_gemm(case.M, case.N, case.K, case.A, case.SFA, case.B, case.SFB,
                                fmt="e2m1")
    rows, cols = [0, 32, 7], [19, 0, 11]
    rp, bp = oracle.mx_gemm_points(case.M, case.N, case.K, case.A, case.SFA, case.B, case.SFB,
                                   rows, cols, fmt="e2m1")
    assert np.array_equal(rp, ref[rows, cols]) and np.array_equal(bp, bound[rows, cols])


def test_mxfp4_quantizer_scale_and_rounding():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 128)).astype(np.float32)
    x[1, 64:96] = 0.0
    packed, scales = si.mxfp4_quantize(x)
    assert packed.shape == (5, 64) and scales.shape == (5, 4)
    xb = x.reshape(5, 4, 32)
    amax = np.abs(xb).max(axis=2)
    X = np.ldexp(1.0, scales.numpy().astype(np.int64) - 127)
    nz = amax > 0
    # the block's absmax lands in [4X, 8X): e2m1's top binade
    assert np.all(4 * X[nz] <= amax[nz]) and np.all(amax[nz] < 8 * X[nz])
    assert X[1, 2] == 1.0
    dec = _unpack4(packed).reshape(5, 4, 32) * X[:, :, None]
    # nearest e2m1 value: within half a step (the step is X/2 below 2X... 2X above 4X)
    step = np.where(np.abs(xb) < 2 * X[:, :, None], 0.5, np.where(np.abs(xb) < 4 * X[:, :, None], 1.0, 2.0)) * X[:, :, None]
    clipped = np.clip(xb, -6 * X[:, :, None], 6 * X[:, :, None])
    assert np.all(np.abs(dec - clipped) <= step / 2 + 1e-30)


def test_grouped_single_group_equals_dense():
    case = si.grouped_case([96], 40, 64, 5)
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    r2, b2 = oracle.gemm(96, 40, 64, case.A, "k", case.B.reshape(40, 64), "k", "bf16")
    assert np.array_equal(ref, r2) and np.array_equal(bound, b2)


def test_grouped_is_concatenation_of_numpy_products_with_empty_groups():
    m_sizes = [3, 0, 5, 1, 0]
    case = si.grouped_case(m_sizes, 6, 16, 6)
    ref, _ = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    a = case.A.to(torch.float64).numpy()
    b = case.B.to(torch.float64).numpy()
    parts = []
    for g, m in enumerate(m_sizes):
        lo = case.m_offsets[g]
        parts.append(a[lo:lo + m] @ b[g].T)
    expect = np.concatenate(parts, axis=0)
    assert ref.shape == (9, 6)
    assert np.allclose(ref, expect, rtol=1e-13, atol=1e-13)
    # Group 2 uses B_2 and nothing else.
    assert np.allclose(ref[3:8], a[3:8] @ b[2].T, rtol=1e-13, atol=1e-13)
