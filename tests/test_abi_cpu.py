"""C-ABI checks that need no GPU: the library loads, exports every function
include/swizzled_gemm.h declares, rejects every invalid argument with the
documented code before touching the GPU, and its LDS byte map equals the
oracle's swizzle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_gemm_swizzled_amd as sg
from oracle import swizzle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swizzled_gemm.h")

NULL, ALIGN, SHAPE, DTYPE, MAJOR, GROUPS = -1, -2, -3, -4, -5, -6
P = 0x10000  # a 16-byte-aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gemm_run", "gemm_strided_run", "grouped_gemm_run", "mx_gemm_run", "mxfp4_gemm_run",
            "mxfp6_gemm_run", "gemm_layout_run", "gemm_layout128_run", "gemm_layout_io_run",
            "gemm_last_error", "gemm_version", "gemm_lds_layout", "gemm_lds_layout_mxfp6",
            "gemm_lds_layout_cblock", "gemm_lds_image"} <= set(names)
    lib = ctypes.CDLL(sg.library_path())
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("kw,code", [
    (dict(swz=4), SHAPE), (dict(swz=32), SHAPE), (dict(swz=-1), SHAPE),
    (dict(M=-1), SHAPE), (dict(D=None), NULL), (dict(A=None), NULL),
    (dict(A=P + 8), ALIGN), (dict(K=60), ALIGN), (dict(d_dtype=sg.SG_E4M3), DTYPE),
    (dict(C=P + 4096, c_dtype=9), DTYPE),
])
def test_gemm_layout_run_rejects(kw, code):
    a = dict(swz=16, M=256, N=256, K=64, A=P, B=P, C=None, c_dtype=0, D=P,
             d_dtype=sg.SG_F32)
    a.update(kw)
    rc = sg.gemm_layout_run(a["swz"], a["M"], a["N"], a["K"], a["A"], a["B"], a["C"],
                            a["c_dtype"], a["D"], a["d_dtype"], None)
    assert rc == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("gemm_layout_run")


def _strided(**kw):
    a = dict(M=300, N=264, K=136, alpha=1.0, A=P, lda=136, a_major=0, B=P, ldb=136, b_major=0,
             ab=sg.SG_BF16, beta=1.0, C=None, ldc=264, c_dtype=0, D=P, ldd=264,
             d_dtype=sg.SG_F32)
    a.update(kw)
    return sg.gemm_strided_run(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                               a["a_major"], a["B"], a["ldb"], a["b_major"], a["ab"],
                               a["beta"], a["C"], a["ldc"], a["c_dtype"], a["D"], a["ldd"],
                               a["d_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lda=128), SHAPE), (dict(ldb=100), SHAPE), (dict(ldd=256), SHAPE),
    (dict(C=P + 8192, c_dtype=sg.SG_BF16, ldc=200), SHAPE),
    (dict(a_major=1, lda=296), SHAPE),            # MN-major A needs lda >= M = 300
    (dict(lda=140), ALIGN), (dict(ldb=137), ALIGN), (dict(ldd=266), ALIGN),
    (dict(C=P + 8192, c_dtype=sg.SG_BF16, ldc=268), ALIGN),
    (dict(C=P, c_dtype=sg.SG_F32, ldc=272), DTYPE),  # in place needs ldc == ldd
    (dict(A=None), NULL), (dict(M=-1), SHAPE), (dict(a_major=7), MAJOR),
    (dict(N=262), SHAPE), (dict(N=261, M=0), SHAPE),  # D is written 4 columns at a time
    # a K-major operand needs K % 8 == 0 (the loaders move whole 16-byte
    # chunks, so K = 100 with lda = 104 would read elements 100..103 from the
    # row padding)
    (dict(K=100, lda=104, ldb=104), SHAPE),
    (dict(K=100, lda=304, a_major=1, ldb=104), SHAPE),
    (dict(K=100, lda=104, ldb=264, b_major=1), SHAPE),
])
def test_gemm_strided_run_rejects(kw, code):
    rc = _strided(**kw)
    assert rc == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("gemm_strided_run")


def test_gemm_strided_run_k_not_multiple_of_8_needs_mn_major_operands():
    # Both operands MN-major: K indexes rows, which the loaders bound row by
    # row, so K = 100 passes validation (the call then fails only at the
    # launch, which needs a GPU).
    rc = _strided(K=100, lda=304, a_major=1, ldb=264, b_major=1)
    assert rc != SHAPE, sg.gemm_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(ops=8), SHAPE), (dict(ops=-1), SHAPE), (dict(out=2), SHAPE),
    (dict(d_dtype=sg.SG_F32), DTYPE), (dict(C=P + 4096, c_dtype=sg.SG_F32), DTYPE),
    (dict(M=-1), SHAPE), (dict(A=None), NULL), (dict(K=60), ALIGN),
])
def test_gemm_layout_io_run_rejects(kw, code):
    a = dict(ops=16, out=1, M=256, N=256, K=64, A=P, B=P, C=None, c_dtype=0, D=P,
             d_dtype=sg.SG_BF16)
    a.update(kw)
    rc = sg.gemm_layout_io_run(a["ops"], a["out"], a["M"], a["N"], a["K"], a["A"], a["B"],
                               a["C"], a["c_dtype"], a["D"], a["d_dtype"], None)
    assert rc == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("gemm_layout_io_run")


def test_cblock_layout_rejects_null():
    assert sg.load().gemm_lds_layout_cblock(None) == NULL
    assert sg.gemm_last_error().startswith("gemm_lds_layout_cblock")


def test_gemm_strided_run_unread_operands_may_be_null():
    # alpha == 0 reads neither A nor B, beta == 0 does not read C: no
    # launch happens for M = 0, and the checks that remain pass.
    assert _strided(M=0, alpha=0.0, A=None, B=None) == 0
    assert _strided(N=0, beta=0.0, C=P + 3, c_dtype=sg.SG_F32) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(layout=4), SHAPE), (dict(layout=-2), SHAPE), (dict(M=-1), SHAPE), (dict(D=None), NULL),
    (dict(A=P + 8), ALIGN), (dict(K=60), ALIGN), (dict(d_dtype=sg.SG_E4M3), DTYPE),
])
def test_gemm_layout128_run_rejects(kw, code):
    a = dict(layout=sg.SG_LAYOUT_PAD16, M=256, N=256, K=64, A=P, B=P, C=None, c_dtype=0, D=P,
             d_dtype=sg.SG_F32)
    a.update(kw)
    rc = sg.gemm_layout128_run(a["layout"], a["M"], a["N"], a["K"], a["A"], a["B"], a["C"],
                               a["c_dtype"], a["D"], a["d_dtype"], None)
    assert rc == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("gemm_layout128_run")


def test_gemm_layout128_run_empty_is_ok():
    for layout in (0, 8, 16, sg.SG_LAYOUT_PAD16):
        assert sg.gemm_layout128_run(layout, 0, 256, 64, P, P, None, 0, P, sg.SG_F32, None) == 0


def test_gemm_layout_run_empty_is_ok():
    for swz in (0, 8, 16):
        assert sg.gemm_layout_run(swz, 0, 256, 64, P, P, None, 0, P, sg.SG_F32, None) == 0


def test_version_and_empty_error():
    assert "gfx950" in sg.gemm_version()


def _gemm(**kw):
    a = dict(M=256, N=256, K=64, A=P, a_major=0, B=P, b_major=0, ab_dtype=sg.SG_BF16,
             C=None, c_dtype=0, D=P, d_dtype=sg.SG_F32, stream=None)
    a.update(kw)
    return sg.gemm_run(a["M"], a["N"], a["K"], a["A"], a["a_major"], a["B"], a["b_major"],
                       a["ab_dtype"], a["C"], a["c_dtype"], a["D"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), SHAPE), (dict(K=-5), SHAPE),
    (dict(ab_dtype=sg.SG_F32), DTYPE), (dict(ab_dtype=9), DTYPE),
    (dict(d_dtype=sg.SG_E4M3), DTYPE), (dict(C=P + 4096, c_dtype=7), DTYPE),
    (dict(C=P, c_dtype=sg.SG_BF16, d_dtype=sg.SG_F32), DTYPE),  # C == D, other dtype
    (dict(a_major=2), MAJOR), (dict(b_major=-1), MAJOR),
    (dict(D=None), NULL), (dict(A=None), NULL), (dict(B=None), NULL),
    (dict(A=P + 8), ALIGN), (dict(B=P + 2), ALIGN), (dict(D=P + 4), ALIGN),
    (dict(C=P + 4104, c_dtype=sg.SG_BF16), ALIGN),
    (dict(K=60), ALIGN),                      # 120-byte K-major rows
    (dict(M=100, a_major=1), ALIGN),          # 200-byte MN-major A rows
    (dict(N=100, b_major=1), ALIGN),
])
def test_gemm_run_rejects(kw, code):
    rc = _gemm(**kw)
    assert rc == code, (kw, rc, sg.gemm_last_error())
    assert sg.gemm_last_error()


def test_gemm_run_bf16_output_pitch():
    assert _gemm(N=260, d_dtype=sg.SG_BF16) == ALIGN   # 520-byte rows


def test_gemm_run_oversized_panel():
    # MN-major A of 2^30 elements spans 2^31 bytes.
    assert _gemm(M=1 << 15, K=1 << 15, a_major=1) == SHAPE


def test_empty_problems_are_noops_without_pointers():
    assert _gemm(M=0, A=None, B=None, D=None) == sg.SG_OK
    assert _gemm(N=0, A=None, B=None, D=None) == sg.SG_OK


def _grouped(**kw):
    a = dict(G=2, offs=[0, 128, 256], N=256, K=64, A=P, a_major=0, B=P, b_major=0,
             ab_dtype=sg.SG_BF16, D=P, d_dtype=sg.SG_BF16)
    a.update(kw)
    return sg.grouped_gemm_run(a["G"], a["offs"], a["N"], a["K"], a["A"], a["a_major"],
                               a["B"], a["b_major"], a["ab_dtype"], a["D"], a["d_dtype"],
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=0, offs=[0]), GROUPS), (dict(G=257, offs=list(range(258))), GROUPS),
    (dict(offs=[1, 128, 256]), GROUPS), (dict(offs=[0, 200, 100]), GROUPS),
    (dict(offs=None), NULL), (dict(D=None), NULL), (dict(A=None), NULL),
    (dict(a_major=1), MAJOR), (dict(b_major=1), MAJOR),
    (dict(ab_dtype=sg.SG_E4M3), DTYPE), (dict(d_dtype=0), DTYPE),
    (dict(K=12), ALIGN), (dict(N=-1), SHAPE),
])
def test_grouped_rejects(kw, code):
    assert _grouped(**kw) == code, sg.gemm_last_error()


def test_grouped_all_empty_is_noop():
    assert _grouped(offs=[0, 0, 0], A=None, B=None, D=None) == sg.SG_OK


def test_grouped_accepts_the_largest_group_count():
    # SG_MAX_GROUPS offsets travel by value in the kernel arguments; G = 256
    # passes every check (all groups empty, so nothing is launched).
    assert sg.SG_MAX_GROUPS == 256
    G = sg.SG_MAX_GROUPS
    assert _grouped(G=G, offs=[0] * (G + 1)) == sg.SG_OK, sg.gemm_last_error()
    assert _grouped(G=G + 1, offs=[0] * (G + 2)) == GROUPS
    # a decrease at the last group is still seen
    assert _grouped(G=G, offs=[0] * G + [-1]) == GROUPS


def _mx(**kw):
    a = dict(M=256, N=256, K=256, A=P, SFA=P, B=P, SFB=P, D=P, d_dtype=sg.SG_BF16)
    a.update(kw)
    return sg.mx_gemm_run(a["M"], a["N"], a["K"], a["A"], a["SFA"], a["B"], a["SFB"],
                          a["D"], a["d_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=96), SHAPE), (dict(M=-2), SHAPE), (dict(d_dtype=sg.SG_F16), DTYPE),
    (dict(SFA=None), NULL), (dict(D=None), NULL),
    (dict(SFB=P + 2), ALIGN), (dict(A=P + 8), ALIGN), (dict(N=260), ALIGN),
])
def test_mx_rejects(kw, code):
    assert _mx(**kw) == code, sg.gemm_last_error()


def _mx4(**kw):
    a = dict(M=256, N=256, K=512, A=P, SFA=P, B=P, SFB=P, D=P, d_dtype=sg.SG_BF16)
    a.update(kw)
    return sg.mxfp4_gemm_run(a["M"], a["N"], a["K"], a["A"], a["SFA"], a["B"], a["SFB"],
                             a["D"], a["d_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=128), SHAPE), (dict(K=384), SHAPE), (dict(N=-1), SHAPE),
    (dict(d_dtype=sg.SG_F16), DTYPE), (dict(d_dtype=sg.SG_E4M3), DTYPE),
    (dict(A=None), NULL), (dict(SFB=None), NULL), (dict(D=None), NULL),
    (dict(B=P + 8), ALIGN), (dict(SFA=P + 1), ALIGN), (dict(N=260), ALIGN),
])
def test_mxfp4_rejects(kw, code):
    assert _mx4(**kw) == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("mxfp4_gemm_run")


def test_mxfp4_empty_is_ok():
    assert _mx4(M=0) == 0 and _mx4(N=0) == 0


def _mx6(**kw):
    a = dict(fmt=sg.SG_E2M3, M=256, N=256, K=512, A=P, SFA=P, B=P, SFB=P, D=P,
             d_dtype=sg.SG_BF16)
    a.update(kw)
    return sg.mxfp6_gemm_run(a["fmt"], a["M"], a["N"], a["K"], a["A"], a["SFA"], a["B"],
                             a["SFB"], a["D"], a["d_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=sg.SG_E4M3), DTYPE), (dict(fmt=6), DTYPE), (dict(fmt=9), DTYPE),
    (dict(K=64), SHAPE), (dict(K=96), SHAPE), (dict(M=-1), SHAPE),
    (dict(K=1 << 24), SHAPE),
    (dict(d_dtype=sg.SG_F16), DTYPE), (dict(d_dtype=sg.SG_E2M3), DTYPE),
    (dict(A=None), NULL), (dict(SFA=None), NULL), (dict(B=None), NULL), (dict(D=None), NULL),
    (dict(A=P + 8), ALIGN), (dict(SFB=P + 2), ALIGN), (dict(D=P + 4), ALIGN),
    (dict(N=260), ALIGN),
])
def test_mxfp6_rejects(kw, code):
    assert _mx6(**kw) == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("mxfp6_gemm_run")


def test_mxfp6_empty_is_ok():
    assert _mx6(M=0) == 0 and _mx6(N=0, fmt=sg.SG_E3M2) == 0
    # K = 0 with M, N > 0 computes D = 0 and reads neither operand (needs a
    # GPU, so only the argument checks are exercised here: NULL operands are
    # accepted when K = 0)
    assert _mx6(M=0, K=0, A=None, B=None, SFA=None, SFB=None) == 0


def _mxb(**kw):
    a = dict(fmt=sg.SG_E4M3, M=256, N=256, K=512, A=P, SFA=P, B=P, SFB=P, D=P,
             d_dtype=sg.SG_BF16)
    a.update(kw)
    return sg.mx_gemm_blocks_run(a["fmt"], a["M"], a["N"], a["K"], a["A"], a["SFA"], a["B"],
                                 a["SFB"], a["D"], a["d_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=sg.SG_BF16), DTYPE), (dict(fmt=9), DTYPE), (dict(fmt=sg.SG_E8M0), DTYPE),
    (dict(K=96), SHAPE), (dict(fmt=sg.SG_E2M1, K=384), SHAPE), (dict(M=-1), SHAPE),
    (dict(d_dtype=sg.SG_F16), DTYPE),
    (dict(A=None), NULL), (dict(SFA=None), NULL), (dict(SFB=None), NULL), (dict(D=None), NULL),
    # the blocks layout is read 16 bytes at a time: 4-byte alignment is not enough
    (dict(SFA=P + 4), ALIGN), (dict(SFB=P + 8), ALIGN), (dict(B=P + 8), ALIGN),
    (dict(N=260), ALIGN),
])
def test_mx_blocks_rejects(kw, code):
    assert _mxb(**kw) == code, sg.gemm_last_error()
    assert sg.gemm_last_error().startswith("mx_gemm_blocks_run")


def test_mx_blocks_empty_is_ok():
    for fmt in (sg.SG_E4M3, sg.SG_E2M1, sg.SG_E2M3, sg.SG_E3M2):
        assert _mxb(fmt=fmt, M=0) == 0 and _mxb(fmt=fmt, N=0) == 0


def test_mx_rows_layout_still_takes_4_byte_aligned_scales():
    # Only the argument checks run (no GPU).  The panel-size check comes after
    # the alignment check: with P + 4 scales the rows layout reaches it
    # (SHAPE), the blocks layout stops at the alignment (ALIGN).
    assert _mx(SFA=P + 4, SFB=P + 4, K=1 << 24) == SHAPE
    assert _mxb(SFA=P + 4, SFB=P + 4, K=1 << 24) == ALIGN
    assert _mxb(K=1 << 24) == SHAPE


@pytest.mark.parametrize("rows,K,nbytes", [
    (64, 512, 1024), (65, 512, 2048), (64, 640, 2048), (0, 512, 0), (100, 128, 2048),
    (8192, 8192, 8192 // 64 * 16 * 1024), (1, 32, 1024),
])
def test_mx_scales_blocks_bytes(rows, K, nbytes):
    assert sg.mx_scales_blocks_bytes(rows, K) == nbytes


@pytest.mark.parametrize("rows,K", [(-1, 512), (64, -32), (64, 48)])
def test_mx_scales_blocks_bytes_rejects(rows, K):
    assert sg.mx_scales_blocks_bytes(rows, K) == SHAPE
    assert sg.gemm_last_error().startswith("mx_scales_blocks_bytes")


@pytest.mark.parametrize("kw,code", [
    (dict(K=96), SHAPE), (dict(rows=-1), SHAPE), (dict(K=-128), SHAPE),
    (dict(SF=None), NULL), (dict(out=None), NULL),
    (dict(SF=P + 2), ALIGN), (dict(out=P + 8), ALIGN),
])
def test_mx_scales_to_blocks_rejects(kw, code):
    a = dict(SF=P, rows=64, K=512, out=P)
    a.update(kw)
    assert sg.mx_scales_to_blocks(a["SF"], a["rows"], a["K"], a["out"], None) == code
    assert sg.gemm_last_error().startswith("mx_scales_to_blocks")


def test_mx_scales_to_blocks_empty_is_ok():
    assert sg.mx_scales_to_blocks(None, 0, 512, None, None) == 0
    assert sg.mx_scales_to_blocks(None, 64, 0, None, None) == 0


def test_mxfp6_layout_is_the_xor_swizzle_with_odd_rows_shifted():
    # Restated from the definition: byte b of row r sits at byte b + 8 of the
    # row when r is odd (and not at the unshifted block position), in the
    # 16-byte unit given by the 128-byte-row XOR map.
    unit = swizzle.lds_tile_map(64, 128, line_bytes=256)
    for e in (32, 5, 0):
        got = sg.gemm_lds_layout_mxfp6(64, e)
        for r in range(64):
            s = 8 if (r % 2 == 1 and r % 32 != e) else 0
            for q in range(12):
                b = 8 * q + s
                assert got[r, q] == unit[r, b // 16] + b % 16, (e, r, q)
    with pytest.raises(sg.GemmError):
        sg.gemm_lds_layout_mxfp6(48)
    with pytest.raises(sg.GemmError):
        sg.gemm_lds_layout_mxfp6(64, 33)


@pytest.mark.parametrize("row_bytes", [64, 128, 256])
@pytest.mark.parametrize("rows", [8, 128, 256])
def test_lds_layout_equals_oracle_swizzle(rows, row_bytes):
    got = sg.gemm_lds_layout(rows, row_bytes)
    want = swizzle.lds_tile_map(rows, row_bytes, line_bytes=256)
    assert np.array_equal(got, want)


def test_lds_layout_rejects():
    with pytest.raises(sg.GemmError):
        sg.gemm_lds_layout(12, 128)
    with pytest.raises(sg.GemmError):
        sg.gemm_lds_layout(8, 96)


def test_lds_image_rejects():
    assert sg.gemm_lds_image(P, 100, 64, 2, 0, 0, 64, P, None) == SHAPE
    assert sg.gemm_lds_image(P, 100, 64, 2, 0, 32, 128, P, None) == SHAPE
    assert sg.gemm_lds_image(None, 100, 64, 2, 0, 0, 128, P, None) == NULL


def test_gemm_plan_rejects_mismatched_shapes():
    import torch
    A = torch.zeros(8, 16, dtype=torch.bfloat16)
    B = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(sg.GemmError):
        sg.gemm_plan(A, B, out=torch.zeros(8, 5))      # out is [M][N] = [8][4]
    with pytest.raises(sg.GemmError):
        sg.gemm_plan(A, torch.zeros(4, 12, dtype=torch.bfloat16), out=torch.zeros(8, 4))
