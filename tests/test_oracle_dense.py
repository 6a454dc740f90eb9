"""Pins of the oracle's dense GEMM and its fp16/bf16 decode (CPU only).

Each check compares the oracle with something other than itself: numpy's
integer / fp64 matmul on logical matrices the test builds (a library routine
on a special case), closed forms (identity, permutation, all-ones, A = 0),
and torch's own bf16/fp16 -> fp64 conversion over every bit pattern.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

pytestmark = []


def _store(logical_rows_by_k: np.ndarray, major: str, dtype: str):
    """logical [R][K] -> storage tensor of the given majorness/dtype."""
    x = logical_rows_by_k if major == "k" else logical_rows_by_k.T
    return si.to_dtype(np.ascontiguousarray(x.astype(np.float32)), dtype)


def _store_b(b_kn: np.ndarray, major: str, dtype: str):
    """logical B [K][N] -> storage ([N][K] if K-major else [K][N])."""
    x = b_kn.T if major == "k" else b_kn
    return si.to_dtype(np.ascontiguousarray(x.astype(np.float32)), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_all_bit_patterns_match_torch(dtype):
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    x = bits.view(tdt)
    ours = oracle.decode(dtype, x)
    theirs = x.to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])


@pytest.mark.parametrize("a_major,b_major", list(itertools.product(["k", "mn"], repeat=2)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 4), (4, 1, 3), (3, 4, 2), (5, 7, 9)])
def test_integer_inputs_match_numpy_exactly(M, N, K, dtype, a_major, b_major):
    seed = M * 100 + N * 10 + K
    a = si.integer_valued((M, K), seed)
    b = si.integer_valued((K, N), seed + 1)
    c = si.integer_valued((M, N), seed + 2)
    A = _store(a, a_major, dtype)
    B = _store_b(b, b_major, dtype)
    C = si.to_dtype(c, "f32")
    ref, bound = oracle.gemm(M, N, K, A, a_major, B, b_major, dtype, C, "f32")
    expect = a.astype(np.int64) @ b.astype(np.int64) + c.astype(np.int64)
    assert np.array_equal(ref, expect.astype(np.float64))
    expect_bound = np.abs(a.astype(np.int64)) @ np.abs(b.astype(np.int64)) + np.abs(c)
    assert np.array_equal(bound, expect_bound.astype(np.float64))


@pytest.mark.parametrize("a_major,b_major", list(itertools.product(["k", "mn"], repeat=2)))
def test_random_bf16_matches_numpy_fp64(a_major, b_major):
    M, N, K = 37, 29, 131
    rng = np.random.default_rng(7)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    A = _store(a, a_major, "bf16")
    B = _store_b(b, b_major, "bf16")
    ref, bound = oracle.gemm(M, N, K, A, a_major, B, b_major, "bf16")
    # The logical operands as torch decodes them, multiplied by numpy.
    al = (A.to(torch.float64).numpy() if a_major == "k" else A.to(torch.float64).numpy().T)
    bl = (B.to(torch.float64).numpy().T if b_major == "k" else B.to(torch.float64).numpy())
    expect = al @ bl
    assert np.all(np.abs(ref - expect) <= 1e-12 * (np.abs(al) @ np.abs(bl)))
    assert np.allclose(bound, np.abs(al) @ np.abs(bl), rtol=1e-13, atol=0)


def test_identity_gives_b_exactly():
    n, N = 16, 24
    a = np.eye(n, dtype=np.float32)
    rng = np.random.default_rng(3)
    b = rng.standard_normal((n, N)).astype(np.float32)
    A = _store(a, "k", "bf16")
    B = _store_b(b, "mn", "bf16")
    ref, _ = oracle.gemm(n, N, n, A, "k", B, "mn", "bf16")
    assert np.array_equal(ref, B.to(torch.float64).numpy())


def test_permutation_permutes_rows_exactly():
    n, N = 12, 20
    perm = np.random.default_rng(5).permutation(n)
    a = np.zeros((n, n), dtype=np.float32)
    a[np.arange(n), perm] = 1.0
    b = np.random.default_rng(6).standard_normal((n, N)).astype(np.float32)
    A = _store(a, "mn", "f16")
    B = _store_b(b, "k", "f16")
    ref, _ = oracle.gemm(n, N, n, A, "mn", B, "k", "f16")
    bl = B.to(torch.float64).numpy().T
    assert np.array_equal(ref, bl[perm])


def test_all_ones_gives_k():
    M, N, K = 5, 6, 77
    A = torch.ones(M, K, dtype=torch.bfloat16)
    B = torch.ones(N, K, dtype=torch.bfloat16)
    ref, bound = oracle.gemm(M, N, K, A, "k", B, "k", "bf16")
    assert np.all(ref == K) and np.all(bound == K)


def test_zero_a_gives_c_and_null_c_equals_zero_c():
    M, N, K = 9, 8, 16
    A = torch.zeros(M, K, dtype=torch.bfloat16)
    B = si.to_bf16(np.random.default_rng(1).standard_normal((N, K)).astype(np.float32))
    C = si.to_bf16(np.random.default_rng(2).standard_normal((M, N)).astype(np.float32))
    ref, bound = oracle.gemm(M, N, K, A, "k", B, "k", "bf16", C, "bf16")
    assert np.array_equal(ref, C.to(torch.float64).numpy())
    assert np.array_equal(bound, np.abs(C.to(torch.float64).numpy()))
    A2 = si.to_bf16(np.random.default_rng(3).standard_normal((M, K)).astype(np.float32))
    r_null, _ = oracle.gemm(M, N, K, A2, "k", B, "k", "bf16")
    r_zero, _ = oracle.gemm(M, N, K, A2, "k", B, "k", "bf16",
                            torch.zeros(M, N, dtype=torch.bfloat16), "bf16")
    assert np.array_equal(r_null, r_zero)


def test_k_zero_gives_c():
    M, N = 3, 4
    C = torch.arange(12, dtype=torch.float32).reshape(M, N)
    ref, bound = oracle.gemm(M, N, 0, torch.empty(0, dtype=torch.bfloat16), "k",
                             torch.empty(0, dtype=torch.bfloat16), "k", "bf16", C, "f32")
    assert np.array_equal(ref, C.numpy().astype(np.float64))


def test_points_agree_with_full_and_threads_do_not_matter():
    case = si.dense_case(70, 50, 96, 11, ab_dtype="bf16", a_major="mn",
                         b_major="k", with_c=True, c_dtype="f32")
    ref1, b1 = oracle.gemm(case.M, case.N, case.K, case.A, "mn", case.B, "k",
                           "bf16", case.C, "f32", nthreads=1)
    ref8, b8 = oracle.gemm(case.M, case.N, case.K, case.A, "mn", case.B, "k",
                           "bf16", case.C, "f32", nthreads=8)
    assert np.array_equal(ref1, ref8) and np.array_equal(b1, b8)
    rows = [0, 69, 13, 42]
    cols = [0, 49, 7, 30]
    rp, bp = oracle.gemm_points(case.M, case.N, case.K, case.A, "mn", case.B,
                                "k", "bf16", rows, cols, case.C, "f32")
    assert np.array_equal(rp, ref1[rows, cols])
    assert np.array_equal(bp, b1[rows, cols])


def test_integer_valued_large_k_exact():
    # |a|,|b| <= 4 so every partial sum of K <= 8192 terms is an integer
    # below 2^24: any correct summation order gives the exact result.
    M, N, K = 4, 5, 8192
    a = si.integer_valued((M, K), 21)
    b = si.integer_valued((K, N), 22)
    ref, _ = oracle.gemm(M, N, K, _store(a, "k", "bf16"), "k",
                         _store_b(b, "k", "bf16"), "k", "bf16")
    assert np.array_equal(ref, (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64))


def test_rejects_bad_arguments():
    A = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, A, "k", A, "k", "f32")
    with pytest.raises(ValueError):
        oracle.gemm_points(4, 4, 4, A, "k", A, "k", "bf16", [4], [0])
