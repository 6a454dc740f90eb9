"""Pins of the strided, scaled oracle gemm_ex (CPU): D = alpha*A*B + beta*C
read from padded storage.  Integer values make every product and sum exact,
so numpy's int64 matmul of the logical matrices is the expected result; the
padding holds NaN, so reading a wrong element shows up as NaN."""
import numpy as np
import pytest

import oracle

NAN_BF16 = np.int16(0x7FC0)
NAN_F32 = np.float32(np.nan)


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    # Integers in [-8, 8] are exact in bf16: the upper 16 bits of their fp32.
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


def _padded(logical: np.ndarray, ld: int, fill) -> np.ndarray:
    rows, cols = logical.shape
    buf = np.full((rows, ld), fill, dtype=logical.dtype)
    buf[:, :cols] = logical
    return buf


@pytest.mark.parametrize("a_major", ["k", "mn"])
@pytest.mark.parametrize("b_major", ["k", "mn"])
def test_strided_scaled_matches_int64_matmul(a_major, b_major):
    rng = np.random.default_rng(5)
    M, N, K = 37, 29, 43
    a = rng.integers(-4, 5, (M, K))
    b = rng.integers(-4, 5, (N, K))
    c = rng.integers(-8, 9, (M, N))
    alpha, beta = 2.0, -3.0
    A_log = a if a_major == "k" else a.T          # stored [M][K] or [K][M]
    B_log = b if b_major == "k" else b.T          # stored [N][K] or [K][N]
    lda, ldb, ldc = A_log.shape[1] + 5, B_log.shape[1] + 3, N + 7
    A = _padded(_bf16_bits(A_log), lda, NAN_BF16)
    B = _padded(_bf16_bits(B_log), ldb, NAN_BF16)
    C = _padded(c.astype(np.float32), ldc, NAN_F32)
    ref, bound = oracle.gemm_ex(M, N, K, alpha, A, lda, a_major, B, ldb, b_major, "bf16",
                                beta, C, ldc, "f32")
    want = 2 * (a @ b.T) - 3 * c
    assert np.array_equal(ref, want.astype(np.float64))
    assert np.array_equal(bound, (2 * (np.abs(a) @ np.abs(b).T) + 3 * np.abs(c)).astype(np.float64))


def test_alpha_zero_reads_neither_a_nor_b():
    M, N, K = 5, 6, 7
    A = np.full((M, K), NAN_BF16)
    B = np.full((N, K), NAN_BF16)
    c = np.arange(M * N, dtype=np.float32).reshape(M, N)
    ref, _ = oracle.gemm_ex(M, N, K, 0.0, A, K, "k", B, K, "k", "bf16", 0.5, c, N, "f32")
    assert np.array_equal(ref, 0.5 * c.astype(np.float64))


def test_beta_zero_does_not_read_c():
    M, N, K = 4, 8, 6
    a = np.ones((M, K), dtype=np.int64)
    b = np.ones((N, K), dtype=np.int64)
    C = np.full((M, N), NAN_F32)
    ref, _ = oracle.gemm_ex(M, N, K, -1.5, _bf16_bits(a), K, "k", _bf16_bits(b), K, "k",
                            "bf16", 0.0, C, N, "f32")
    assert np.array_equal(ref, np.full((M, N), -1.5 * K))


def test_packed_unit_scales_equal_plain_gemm():
    # gemm_ex with packed leading dimensions and alpha = beta = 1 is gemm's
    # definition: identical values (both exact here).
    rng = np.random.default_rng(6)
    M, N, K = 20, 24, 16
    a, b = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (N, K))
    c = rng.integers(-5, 6, (M, N)).astype(np.float32)
    r1, _ = oracle.gemm_ex(M, N, K, 1.0, _bf16_bits(a), K, "k", _bf16_bits(b), K, "k", "bf16",
                           1.0, c, N, "f32")
    r2, _ = oracle.gemm(M, N, K, _bf16_bits(a), "k", _bf16_bits(b), "k", "bf16", C=c,
                        c_dtype="f32")
    assert np.array_equal(r1, r2)


def test_rejects_short_leading_dimensions():
    A = np.zeros((4, 8), dtype=np.int16)
    with pytest.raises(ValueError):
        oracle.gemm_ex(4, 4, 8, 1.0, A, 7, "k", A, 8, "k", "bf16", 0.0)
