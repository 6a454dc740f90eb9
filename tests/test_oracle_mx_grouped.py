"""Pins of the oracle's block-scaled (MX) and grouped GEMMs (CPU only).

MX: the e4m3 / e8m0 decode is checked on all 256 codes against torch's
float8_e4m3fn / float8_e8m0fnu conversions and against closed-form values;
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
