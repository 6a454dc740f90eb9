"""The torch wrappers' argument checks, which run before any pointer reaches
the C ABI: a transposed or expanded view, a C or out of the wrong shape, a
grouped A whose rows disagree with the offsets, mismatched K or dtypes, and
tensors that are not on one CUDA device all raise GemmError with the code of
the matching C error.  The device check comes last, so every other check is
exercised here on CPU tensors."""
import pytest
import torch

import dense_gemm_swizzled_amd as sg

NULL, ALIGN, SHAPE, DTYPE, MAJOR, GROUPS = -1, -2, -3, -4, -5, -6


def _code(fn, *a, **kw):
    with pytest.raises(sg.GemmError) as e:
        fn(*a, **kw)
    return e.value.code


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_gemm_rejects_a_transposed_view():
    # sg.gemm(X.t(), W) used to read X's storage as if it were [M][K].
    X, W = bf(16, 8), bf(4, 16)
    assert _code(sg.gemm, X.t(), W) == ALIGN


def test_gemm_rejects_an_expanded_view():
    A = bf(1, 16).expand(8, 16)
    assert _code(sg.gemm, A, bf(4, 16)) == ALIGN


@pytest.mark.parametrize("fn", [sg.gemm, sg.gemm_plan])
def test_gemm_rejects_wrong_c_and_out(fn):
    A, B = bf(8, 16), bf(4, 16)
    out = torch.zeros(8, 4)
    assert _code(fn, A, B, C=torch.zeros(8, 5), out=out) == SHAPE
    assert _code(fn, A, B, C=torch.zeros(4, 8).t(), out=out) == ALIGN
    assert _code(fn, A, B, out=torch.zeros(8, 3)) == SHAPE
    assert _code(fn, A, B, out=torch.zeros(4, 8).t()) == ALIGN
    assert _code(fn, A, B, C=torch.zeros(8, 4, dtype=torch.int32), out=out) == DTYPE


def test_gemm_rejects_k_and_dtype_mismatch():
    assert _code(sg.gemm, bf(8, 16), bf(4, 12)) == SHAPE
    assert _code(sg.gemm, bf(8, 16), torch.zeros(4, 16, dtype=torch.float16)) == DTYPE
    assert _code(sg.gemm, torch.zeros(8, 16), torch.zeros(4, 16)) == DTYPE
    assert _code(sg.gemm, bf(16, 8), bf(16, 4), a_major="mn", b_major="x") == MAJOR
    # MN-major shapes are read transposed: A [K][M], B [K][N]
    assert _code(sg.gemm, bf(16, 8), bf(12, 4), a_major="mn", b_major="mn") == SHAPE


def test_gemm_rejects_cpu_tensors_last():
    # Every shape and layout check passes: only the device is wrong.
    assert _code(sg.gemm, bf(8, 16), bf(4, 16), C=torch.zeros(8, 4),
                 out=torch.zeros(8, 4)) == NULL


def test_gemm_strided_checks():
    A = bf(8, 24)[:, :16]          # padded rows: allowed
    B = bf(4, 16)
    assert _code(sg.gemm_strided, A, B) == NULL              # only the device is wrong
    assert _code(sg.gemm_strided, bf(16, 8).t(), B) == ALIGN  # column stride != 1
    assert _code(sg.gemm_strided, A, B, C=torch.zeros(8, 5)) == SHAPE
    assert _code(sg.gemm_strided, A, B, out=torch.zeros(8, 6)[:, :5]) == SHAPE
    assert _code(sg.gemm_strided, bf(2, 8, 16), B) == SHAPE


def test_grouped_gemm_checks():
    B = bf(3, 8, 16)                       # G = 3, N = 8, K = 16
    offs = [0, 4, 4, 10]
    A = bf(10, 16)
    assert _code(sg.grouped_gemm, A, B, offs) == NULL       # only the device is wrong
    assert _code(sg.grouped_gemm, bf(9, 16), B, offs) == SHAPE   # rows != offsets[-1]
    assert _code(sg.grouped_gemm, bf(10, 12), B, offs) == SHAPE  # K differs
    assert _code(sg.grouped_gemm, A, B, [0, 4, 10]) == GROUPS    # G+1 offsets needed
    assert _code(sg.grouped_gemm, A, bf(24, 16), offs) == SHAPE  # B must be [G][N][K]
    assert _code(sg.grouped_gemm, A, B, offs, out=torch.zeros(10, 9)) == SHAPE
    assert _code(sg.grouped_gemm, bf(16, 10).t(), B, offs) == ALIGN


def u8(*shape):
    return torch.zeros(*shape, dtype=torch.uint8)


@pytest.mark.parametrize("fn,row_bytes,kw", [
    (sg.mx_gemm, 256, {}), (sg.mxfp4_gemm, 128, {}), (sg.mxfp6_gemm, 192, {}),
    (sg.mxfp6_gemm, 192, {"fmt": "e3m2"}),
])
def test_block_scaled_checks(fn, row_bytes, kw):
    K = 256
    A, B = u8(8, row_bytes), u8(4, row_bytes)
    SFA, SFB = u8(8, K // 32), u8(4, K // 32)
    assert _code(fn, A, SFA, B, SFB, **kw) == NULL          # only the device is wrong
    assert _code(fn, A, u8(8, 7), B, SFB, **kw) == SHAPE     # SFA must be [M][K/32]
    assert _code(fn, A, SFA, B, u8(5, 8), **kw) == SHAPE     # SFB must be [N][K/32]
    assert _code(fn, A, SFA, u8(4, row_bytes + 16), SFB, **kw) == SHAPE  # row bytes differ
    assert _code(fn, A, SFA, B, SFB, out=torch.zeros(8, 5), **kw) == SHAPE
    assert _code(fn, A.float(), SFA, B, SFB, **kw) == DTYPE
    assert _code(fn, u8(row_bytes, 8).t(), SFA, B, SFB, **kw) == ALIGN


def test_mxfp6_rejects_unknown_format():
    assert _code(sg.mxfp6_gemm, u8(8, 192), u8(8, 8), u8(4, 192), u8(4, 8), fmt="e4m3") == DTYPE


def u8(*shape):
    return torch.zeros(*shape, dtype=torch.uint8)


def test_mx_scales_blocks_checks():
    assert _code(sg.mx_scales_blocks, torch.zeros(64, 16)) == DTYPE
    assert _code(sg.mx_scales_blocks, u8(64)) == SHAPE
    assert _code(sg.mx_scales_blocks, u8(16, 64).t()) == ALIGN
    assert _code(sg.mx_scales_blocks, u8(64, 16), out=u8(1000)) == SHAPE
    assert _code(sg.mx_scales_blocks, u8(64, 16), out=u8(1024, 1)) == SHAPE
    # every other check passes: only the device is wrong
    assert _code(sg.mx_scales_blocks, u8(64, 16), out=u8(1024)) == NULL


def test_mx_gemm_blocks_checks():
    M, N, K = 64, 32, 512
    A, B = u8(M, K), u8(N, K)
    sfa, sfb = u8(sg.mx_scales_blocks_bytes(M, K)), u8(sg.mx_scales_blocks_bytes(N, K))
    assert _code(sg.mx_gemm_blocks, A, sfa, B, sfb, fmt="e5m2") == DTYPE
    assert _code(sg.mx_gemm_blocks, A, u8(M, K // 32), B, sfb) == SHAPE  # rows layout
    assert _code(sg.mx_gemm_blocks, A, u8(1000), B, sfb) == SHAPE
    assert _code(sg.mx_gemm_blocks, A, sfa, u8(N, K - 16), sfb) == SHAPE
    assert _code(sg.mx_gemm_blocks, A.float(), sfa, B, sfb) == DTYPE
    assert _code(sg.mx_gemm_blocks, A, sfa, B, sfb, out=torch.zeros(M, N + 1)) == SHAPE
    # e2m1: two elements a byte, so the same bytes hold K = 1024
    sfa4 = u8(sg.mx_scales_blocks_bytes(M, 2 * K))
    sfb4 = u8(sg.mx_scales_blocks_bytes(N, 2 * K))
    assert _code(sg.mx_gemm_blocks, A, sfa, B, sfb, fmt="e2m1") == SHAPE
    assert _code(sg.mx_gemm_blocks, A, sfa4, B, sfb4, fmt="e2m1") == NULL
    assert _code(sg.mx_gemm_blocks, A, sfa, B, sfb) == NULL
