"""GPU parity for every kernel instantiation the C ABI can reach, with the
element types and value ranges the workload tests leave out.

Each test names the kernel it is meant to land on and checks it through
gemm_last_kernel(), so a change of the planner cannot silently move a test
onto another kernel.  Comparisons are element by element against the oracle
(|D - ref| <= tau * (sum|a*b| + |c|), tau = 1e-4 for fp32 and 8e-3 for
16-bit outputs) or exact where integer-valued inputs make every partial sum
exact in fp32.

* fp16 operands on the 256x256 ping-pong (K-major, MN-major A, MN-major B,
  both), on the 128x128 two-stage and five-stage kernels, on the 64x64
  eight-stage ring and on both grouped kernels;
* MXFP8 over the whole e4m3 code range (subnormals and magnitudes up to
  448), and e8m0 scale byte 255 (NaN), which must make exactly its own
  row's (or column's) outputs NaN;
* more than 128 groups, with empty groups, on both grouped kernels.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_swizzled_amd as sg
import oracle
import synth_inputs as si
from tests._tol import check_close, tau_mx_f32

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(f"[gpu-kernels] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load()
    return torch.device("cuda:0")


def _np(d):
    return d.float().cpu().numpy().astype(np.float64)


def _to16(x: np.ndarray, ab: str) -> torch.Tensor:
    return si.to_dtype(x, ab)


def _ops(a, b, ab, a_major, b_major):
    A, B = _to16(a, ab), _to16(b, ab)
    A = A if a_major == "k" else A.t().contiguous()
    B = B if b_major == "k" else B.t().contiguous()
    return A, B


def _exact(dev, M, N, K, ab, a_major, b_major, seed, kernel):
    a = si.integer_valued((M, K), seed)
    b = si.integer_valued((N, K), seed + 1)
    A, B = _ops(a, b, ab, a_major, b_major)
    d = sg.gemm(A.to(dev), B.to(dev), a_major=a_major, b_major=b_major,
                out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kernel), sg.gemm_last_kernel()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


# ------------------------------------------------------------ fp16 dense

@pytest.mark.parametrize("K,c_dtype,d_dtype", [(136, "f16", "f16"), (192, "f16", "f32"),
                                               (192, "bf16", "f16")])
def test_pingpong16_f16_k_major(dev, K, c_dtype, d_dtype):
    # 17 x 17 tiles of 256 with ragged M and N; K = 136 takes the loader with
    # per-load K checks, K = 192 the K-exact loader with the C block brought
    # in by the last loads.
    M, N = 4100, 4104
    case = si.dense_case(M, N, K, 201 + K, ab_dtype="f16", with_c=True, c_dtype=c_dtype,
                         d_dtype=d_dtype, scale=1.0 / np.sqrt(K))
    kern = "pingpong16_gemm_kernel<f16,k,k"
    say(f"{kern}> {M}x{N}x{K} C {c_dtype} D {d_dtype}")
    C = case.C.to(dev)
    d = sg.gemm(case.A.to(dev), case.B.to(dev), C=C, out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    ref, bound = oracle.gemm(M, N, K, case.A, "k", case.B, "k", "f16", case.C, c_dtype)
    check_close(_np(d), ref, bound, "f32" if d_dtype == "f32" else "bf16", kern)


@pytest.mark.parametrize("a_major,b_major", [("mn", "k"), ("k", "mn"), ("mn", "mn")])
def test_pingpong16_f16_mn_major_exact(dev, a_major, b_major):
    _exact(dev, 4104, 4104, 320, "f16", a_major, b_major, 211,
           f"pingpong16_gemm_kernel<f16,{a_major},{b_major}")


@pytest.mark.parametrize("a_major,b_major", [("k", "k"), ("mn", "k"), ("k", "mn"), ("mn", "mn")])
def test_two_stage_128_f16_exact(dev, a_major, b_major):
    # 17 x 16 tiles of 128 (two rounds of the CUs): the two-stage kernel.
    say(f"dense_gemm_kernel<128,f16,{a_major},{b_major}> 2104x2000x1000")
    _exact(dev, 2104, 2000, 1000, "f16", a_major, b_major, 221,
           f"dense_gemm_kernel<128,f16,{a_major},{b_major}")


@pytest.mark.parametrize("a_major,b_major,K,kern", [
    ("k", "k", 1000, "pingpong16_gemm_kernel<f16,k,k"),
    ("mn", "k", 1024, "pingpong16_gemm_kernel<f16,mn,k"),
    ("k", "mn", 1024, "pingpong16_gemm_kernel<f16,k,mn"),
    ("mn", "mn", 1000, "dense_gemm_kernel<128,f16,mn,mn"),
])
def test_partial_round_of_256_tiles_f16_exact(dev, a_major, b_major, K, kern):
    # 12 x 12 tiles of 256 (fewer than the CUs) but 24 x 23 of 128 (three
    # rounds): the ping-pong when its loaders take the operands (K-major, or
    # K a multiple of 64), else the two-stage 128x128 kernel.
    say(f"{kern}> 3000x2904x{K}")
    _exact(dev, 3000, 2904, K, "f16", a_major, b_major, 241, kern)


@pytest.mark.parametrize("a_major,b_major", [("k", "k"), ("mn", "k"), ("k", "mn"), ("mn", "mn")])
def test_deep_128_f16_exact(dev, a_major, b_major):
    # 15 x 15 tiles of 128 (one round of CUs): the five-stage ring.
    say(f"deep_gemm_kernel<128,f16,{a_major},{b_major}> 1800x1800x1000")
    _exact(dev, 1800, 1800, 1000, "f16", a_major, b_major, 231,
           f"deep_gemm_kernel<128,f16,{a_major},{b_major}")


@pytest.mark.parametrize("a_major,b_major", [("k", "k"), ("mn", "k"), ("k", "mn"), ("mn", "mn")])
def test_deep_64_f16_exact(dev, a_major, b_major):
    say(f"deep_gemm_kernel<64,f16,{a_major},{b_major}> 520x392x1000")
    _exact(dev, 520, 392, 1000, "f16", a_major, b_major, 241,
           f"deep_gemm_kernel<64,f16,{a_major},{b_major}")


def test_pingpong16_f16_random_with_c(dev):
    # N(0,1)/sqrt(K) fp16 operands over the whole headline shape family
    # (2 x 2 tiles of 256 per CU round), fp16 C and D.
    M, N, K = 4096, 4096, 1024
    case = si.dense_case(M, N, K, 251, ab_dtype="f16", with_c=True, c_dtype="f16",
                         d_dtype="f16", scale=1.0 / np.sqrt(K))
    say(f"pingpong16 f16 {M}x{N}x{K} with fp16 C")
    d = sg.gemm(case.A.to(dev), case.B.to(dev), C=case.C.to(dev), out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("pingpong16_gemm_kernel<f16,k,k")
    ref, bound = oracle.gemm(M, N, K, case.A, "k", case.B, "k", "f16", case.C, "f16")
    check_close(_np(d), ref, bound, "bf16", "pingpong16 f16")


# --------------------------------------------------------- grouped kernels

@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("path", ["256", "128"])
def test_grouped_kernels_dtypes(dev, ab, path):
    # The 256x256 grouped ping-pong (enough tiles) and the 128x128 grouped
    # kernel (few tiles), ragged groups with an empty one.
    if path == "256":
        m_sizes, N, K = [300, 1, 0, 777, 2000, 513, 1200], 4096, 192
        kern = f"pingpong16_grouped_kernel<{ab}"
    else:
        m_sizes, N, K = [0, 37, 128, 0, 300, 1, 256], 264, 200
        kern = f"grouped_gemm_kernel<128,{ab}"
    case = si.grouped_case(m_sizes, N, K, 261, ab_dtype=ab, d_dtype="f32")
    say(f"{kern}> {m_sizes} x {N} x {K}")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, ab)
    check_close(_np(d), ref, bound, "f32", kern)


@pytest.mark.parametrize("G,N,kern", [(256, 1024, "pingpong16_grouped_kernel<bf16"),
                                      (256, 120, "grouped_gemm_kernel<128,bf16"),
                                      (200, 520, "pingpong16_grouped_kernel<bf16")])
def test_grouped_more_than_128_groups(dev, G, N, kern):
    # Up to SG_MAX_GROUPS = 256 groups, a quarter of them empty, sizes off
    # the tile grid: every group's offset and first tile travel in the
    # kernel arguments.
    rng = np.random.default_rng(G + N)
    choices = [0, 0, 1, 5, 37, 100, 128, 200] + ([300] if "pingpong" in kern else [])
    sizes = [int(x) for x in rng.choice(choices, size=G)]
    tiles256 = sum((m + 255) // 256 for m in sizes) * ((N + 255) // 256)
    tiles128 = sum((m + 127) // 128 for m in sizes) * ((N + 127) // 128)
    # the planner's rule: 256x256 tiles fill the CUs, or 128x128 ones need two rounds
    assert (tiles256 >= 256 or tiles128 > 256) == ("pingpong" in kern), (tiles256, tiles128)
    case = si.grouped_case(sizes, N, 128, 271, d_dtype="bf16")
    say(f"{kern}> G={G} N={N} K=128 sum M={case.m_offsets[-1]}")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    check_close(_np(d), ref, bound, "bf16", f"G={G}")


def test_grouped_partial_round_of_256_tiles(dev):
    # 10 x 8 tiles of 256 (fewer than the CUs) but 19 x 16 of 128 (two
    # rounds): the grouped ping-pong, with an empty group and ragged sizes.
    m_sizes, N, K = [700, 650, 0, 800], 2048, 192
    kern = "pingpong16_grouped_kernel<bf16"
    case = si.grouped_case(m_sizes, N, K, 291, d_dtype="f32")
    say(f"{kern}> {m_sizes} x {N} x {K}")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    check_close(_np(d), ref, bound, "f32", kern)


# ------------------------------------------------------ MXFP8 code range

def _e4m3_all_codes(rng, shape):
    """Uniform over the 254 non-NaN e4m3 codes (S.1111.111 is NaN):
    subnormals, zero of both signs and magnitudes up to 448."""
    c = rng.integers(0, 254, shape)
    c = c + (c >= 0x7F)          # skip 0x7F
    return c.astype(np.uint8)    # 254 -> 0xFE; 0xFF never drawn


@pytest.mark.parametrize("M,N,K,kern", [(4100, 4104, 384, "pingpong_mx_kernel<e4m3"),
                                        (2600, 2600, 384, "pingpong_mx_kernel<e4m3"),
                                        (300, 264, 384, "mx_gemm_kernel<128,e4m3")])
def test_mxfp8_full_e4m3_range(dev, M, N, K, kern):
    # 4100 x 4104: 17 x 17 tiles of 256; 2600 x 2600: 11 x 11 tiles of 256
    # but two rounds of 21 x 21 tiles of 128, so the ping-pong too; 300 x 264:
    # the 128x128 kernel.
    rng = np.random.default_rng(M + K)
    A = torch.from_numpy(_e4m3_all_codes(rng, (M, K)))
    B = torch.from_numpy(_e4m3_all_codes(rng, (N, K)))
    # scales 2^-10 .. 2^3 keep every product (up to 448^2 2^6) and sum finite
    SFA = torch.from_numpy(rng.integers(117, 131, (M, K // 32)).astype(np.uint8))
    SFB = torch.from_numpy(rng.integers(117, 131, (N, K // 32)).astype(np.uint8))
    say(f"{kern}> full e4m3 range {M}x{N}x{K}")
    d = sg.mx_gemm(A.to(dev), SFA.to(dev), B.to(dev), SFB.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    ref, bound = oracle.mx_gemm(M, N, K, A, SFA, B, SFB)
    # The scaled MFMA's group alignment may drop up to 7 * 2^-13 of a group's
    # magnitude: the fp32-output tolerance for e4m3 (tests/_tol.py).
    check_close(_np(d), ref, bound, "f32", "full e4m3 range", tau=tau_mx_f32(K))


@pytest.mark.parametrize("M,N,K,kern", [(4096, 4104, 256, "pingpong_mx_kernel<e4m3"),
                                        (300, 264, 256, "mx_gemm_kernel<128,e4m3")])
@pytest.mark.parametrize("d_dtype", ["f32", "bf16"])
def test_mxfp8_nan_scale_poisons_its_row_and_column(dev, M, N, K, kern, d_dtype):
    # e8m0 255 is NaN: a NaN scale of A row r's block b makes all of row r
    # NaN (every column sums over block b), one of B row n all of column n;
    # every other output stays finite and matches the oracle.
    case = si.mx_case(M, N, K, 281)
    SFA, SFB = case.SFA.clone(), case.SFB.clone()
    bad_rows, bad_cols = [0, 257, M - 1], [3, 260, N - 1]
    SFA[257, 1] = 255
    SFA[0, 0] = 255
    SFA[M - 1, K // 32 - 1] = 255
    SFB[3, 2] = 255
    SFB[260, 0] = 255
    SFB[N - 1, K // 32 - 1] = 255
    say(f"{kern}> NaN scales {M}x{N}x{K} D {d_dtype}")
    d = sg.mx_gemm(case.A.to(dev), SFA.to(dev), case.B.to(dev), SFB.to(dev),
                   out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    got = _np(d)
    nan = np.isnan(got)
    want_nan = np.zeros((M, N), dtype=bool)
    want_nan[bad_rows, :] = True
    want_nan[:, bad_cols] = True
    assert np.array_equal(nan, want_nan), (int(nan.sum()), int(want_nan.sum()))
    keep_r = np.setdiff1d(np.arange(M), bad_rows)
    keep_c = np.setdiff1d(np.arange(N), bad_cols)
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB)
    check_close(got[np.ix_(keep_r, keep_c)], ref[np.ix_(keep_r, keep_c)],
                bound[np.ix_(keep_r, keep_c)], d_dtype if d_dtype == "f32" else "bf16",
                "NaN scales, finite outputs", tau=tau_mx_f32(K) if d_dtype == "f32" else None)
