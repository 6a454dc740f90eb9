"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is element by element: |D - ref| <= tau * (sum|a*b| + |c|)
with tau = 1e-4 for fp32 outputs and 8e-3 for bf16/fp16 outputs, no NaN/Inf.
Every comparison covers every output, the 8192^3, grouped 16x4096^2 and
MXFP8 8192^3 workloads included (run at full size in the launch
configuration the bench times; the oracle takes 10-40 s each on the host's
cores), except the MXFP4 and MXFP6 8192^3 runs, which are compared on
sampled outputs the oracle evaluates one by one.  Layout maps are compared
bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_swizzled_amd as sg
import oracle
import synth_inputs as si
from oracle import swizzle
from tests._tol import check_close, tau_mx_f32

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load()
    return torch.device("cuda:0")


def _np(d: torch.Tensor) -> np.ndarray:
    return d.float().cpu().numpy().astype(np.float64)


def run_dense(case: si.DenseCase, dev, out=None, c_override="keep"):
    C = case.C if c_override == "keep" else c_override
    A, B = case.A.to(dev), case.B.to(dev)
    Cd = C.to(dev) if C is not None else None
    if out is None:
        out = torch.empty((case.M, case.N), dtype=DT[case.d_dtype], device=dev)
    sg.gemm(A, B, a_major=case.a_major, b_major=case.b_major, C=Cd, out=out)
    torch.cuda.synchronize()
    return out


def oracle_dense(case: si.DenseCase):
    return oracle.gemm(case.M, case.N, case.K, case.A, case.a_major, case.B,
                       case.b_major, case.ab_dtype, case.C, case.c_dtype)


def sample_points(M, N, n, seed, tile=256):
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n))
    cols = list(rng.integers(0, N, n))
    edges_m = sorted({0, 1, 31, 32, 127, 128, 255, 256, M // 2, M - 2, M - 1} & set(range(M)))
    edges_n = sorted({0, 3, 4, 31, 32, 127, 128, 255, 256, N // 2, N - 4, N - 1} & set(range(N)))
    for r in edges_m:
        for c in edges_n:
            rows.append(r)
            cols.append(c)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


# ------------------------------------------------------------- LDS image

@pytest.mark.parametrize("rows_total,K,eb,row0,k0,tile_rows", [
    (512, 256, 2, 0, 64, 256),     # interior bf16 tile
    (300, 200, 2, 256, 192, 256),  # ragged rows and K tail (16 valid bytes)
    (128, 384, 1, 0, 256, 128),    # fp8 tile of 128 rows
    (200, 64, 2, 128, 0, 128),     # 72 valid rows
])
def test_lds_image_bit_exact(dev, rows_total, K, eb, row0, k0, tile_rows):
    say(f"lds_image rows_total={rows_total} K={K} eb={eb} row0={row0} k0={k0} tile={tile_rows}")
    rng = np.random.default_rng(rows_total + K)
    X = rng.integers(0, 256, (rows_total, K * eb), dtype=np.uint8)
    Xd = torch.from_numpy(X).to(dev)
    out = torch.zeros(tile_rows * 128, dtype=torch.uint8, device=dev)
    rc = sg.gemm_lds_image(Xd.data_ptr(), rows_total, K, eb, row0, k0, tile_rows,
                           out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.gemm_last_error()
    torch.cuda.synchronize()
    tile = np.zeros((tile_rows, 128), dtype=np.uint8)
    r1 = min(rows_total, row0 + tile_rows)
    b0, b1 = k0 * eb, min(K * eb, k0 * eb + 128)
    tile[:r1 - row0, :b1 - b0] = X[row0:r1, b0:b1]
    want = swizzle.lds_image(tile, line_bytes=256)
    assert np.array_equal(out.cpu().numpy(), want)


# -------------------------------------------------------------- dense

def test_single_tile_128x128x32_f16(dev):
    case = si.single_tile(seed=1)
    say(f"{case.name}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32", case.name)


def test_dense_1024_bf16_mn_major_b(dev):
    case = si.dense_1024(seed=2)
    say(f"{case.name}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32", case.name)
    # C = 0 passed explicitly gives the same bits as C = NULL.
    z = torch.zeros(case.M, case.N, dtype=torch.float32)
    d0 = run_dense(case, dev, c_override=z)
    assert torch.equal(d, d0)


@pytest.mark.parametrize("a_major", ["k", "mn"])
@pytest.mark.parametrize("b_major", ["k", "mn"])
@pytest.mark.parametrize("ab", ["bf16", "f16"])
def test_dense_majorness_dtypes_ragged(dev, a_major, b_major, ab):
    M, N, K = 200, 136, 264   # ragged vs 128-row tiles and 64-wide K steps
    case = si.dense_case(M, N, K, 40 + len(a_major) + 2 * len(b_major), ab_dtype=ab,
                         a_major=a_major, b_major=b_major, with_c=True, c_dtype="f32",
                         d_dtype="f32")
    say(f"dense {M}x{N}x{K} {ab} A:{a_major} B:{b_major}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32", "majorness")


@pytest.mark.parametrize("a_major", ["k", "mn"])
@pytest.mark.parametrize("b_major", ["k", "mn"])
def test_dense_128_tiles_ragged(dev, a_major, b_major):
    # 15 x 17 tiles of 128 (8 x 9 of 256): the 128x128 variant; smaller
    # problems take 64x64 tiles, larger ones 256x256.
    M, N, K = 1800, 2056, 200
    case = si.dense_case(M, N, K, 17, a_major=a_major, b_major=b_major, ab_dtype="bf16",
                         with_c=True, c_dtype="bf16", d_dtype="f32", scale=1.0 / np.sqrt(K))
    say(f"dense 128-tile path {M}x{N}x{K} {a_major}/{b_major}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32", "128 tiles")


@pytest.mark.parametrize("tiles", ["64", "128", "128x2"])
def test_dense_deep_ring_integer_exact(dev, tiles):
    # Integer values in [-4, 4] over K = 1000 (16 K tiles, the last partial):
    # every partial sum is exact in fp32, so the result must be bit-exact.
    # The K tiles go round the 64x64 kernel's eight stages twice and the
    # 128x128 kernel's five stages three times; with two rounds of 128x128
    # tiles ("128x2": 272 tiles) the two-stage kernel runs.
    M, N = {"64": (520, 392), "128": (1800, 1800), "128x2": (2100, 2000)}[tiles]
    K = 1000
    a = si.integer_valued((M, K), 95)
    b = si.integer_valued((N, K), 96)
    A, B = si.to_bf16(a), si.to_bf16(b)
    say(f"integer-valued exact, {tiles}-tile deep ring {M}x{N}x{K}")
    d = sg.gemm(A.to(dev), B.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("a_major,b_major", [("mn", "k"), ("k", "mn"), ("mn", "mn")])
def test_dense_128_tiles_deep_ring_mn_major_integer_exact(dev, a_major, b_major):
    # 1800 x 1800: 225 tiles of 128x128, one round of CUs, so the five-stage
    # ring runs; an MN-major operand keeps 256-byte LDS rows per k and is read
    # with transposing reads.  K = 1000: 16 K tiles, the last partial.
    M, N, K = 1800, 1800, 1000
    a = si.integer_valued((M, K), 141)
    b = si.integer_valued((N, K), 142)
    A = si.to_bf16(a) if a_major == "k" else si.to_bf16(a).t().contiguous()
    B = si.to_bf16(b) if b_major == "k" else si.to_bf16(b).t().contiguous()
    say(f"integer-valued exact, 128-tile deep ring {a_major}/{b_major} {M}x{N}x{K}")
    d = sg.gemm(A.to(dev), B.to(dev), a_major=a_major, b_major=b_major,
                out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("a_major,b_major", [("k", "k"), ("mn", "k"), ("k", "mn"), ("mn", "mn")])
@pytest.mark.parametrize("K", [448, 512, 576, 640])
def test_dense_64_tiles_majorness_integer_exact(dev, a_major, b_major, K):
    # 64x64 tiles (520 x 392: 81 tiles) with 7..10 K tiles: from 8 K tiles on
    # (unless both operands are MN-major) the kernel reads fragments two K
    # tiles ahead, with every remainder of its three-way unrolled loop; with 7
    # the one-ahead loop runs.  Integer values keep every sum exact in fp32.
    M, N = 520, 392
    a = si.integer_valued((M, K), 97 + K)
    b = si.integer_valued((N, K), 98 + K)
    A, B = si.to_bf16(a), si.to_bf16(b)
    A = A if a_major == "k" else A.t().contiguous()
    B = B if b_major == "k" else B.t().contiguous()
    say(f"integer-valued exact, 64-tile {M}x{N}x{K} {a_major}/{b_major}")
    d = sg.gemm(A.to(dev), B.to(dev), a_major=a_major, b_major=b_major, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("c_dtype,d_dtype", [(None, "bf16"), ("bf16", "bf16"),
                                             ("f16", "f16"), ("f32", "bf16"),
                                             ("bf16", "f32")])
def test_dense_epilogue_dtypes(dev, c_dtype, d_dtype):
    M, N, K = 136, 264, 72
    case = si.dense_case(M, N, K, 7, ab_dtype="bf16", with_c=c_dtype is not None,
                         c_dtype=c_dtype or "bf16", d_dtype=d_dtype)
    say(f"epilogue C={c_dtype} D={d_dtype}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32" if d_dtype == "f32" else "bf16", "epilogue")


@pytest.mark.parametrize("K", [136, 192])
def test_dense_256_tiles_ragged(dev, K):
    # 17 x 17 tiles of 256 -> the 256x256 variant, ragged in M and N (the last
    # tile row has 4 valid rows: its second wave group skips its MFMAs); K =
    # 136 takes the loader with per-load K checks, K = 192 (a multiple of 64)
    # the loader with fixed row offsets.
    M, N = 4100, 4104
    case = si.dense_case(M, N, K, 11, ab_dtype="bf16", with_c=True, c_dtype="bf16",
                         d_dtype="bf16", scale=1.0 / np.sqrt(K))
    say(f"dense 256-tile path {M}x{N}x{K}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "bf16", "256 tiles")


@pytest.mark.parametrize("K", [8, 64])
def test_dense_256_tiles_single_k_tile(dev, K):
    # 256x256 tiles with one (partial or whole) K tile: the ring's prologue
    # already covers every load and the rest are zero-filled.
    M, N = 4096, 4352
    case = si.dense_case(M, N, K, 12 + K, ab_dtype="bf16", with_c=True, c_dtype="f32",
                         d_dtype="f32", scale=1.0 / np.sqrt(K))
    say(f"dense 256-tile path {M}x{N}x{K}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "f32", f"256 tiles K={K}")


def test_layout_variants_bit_identical(dev):
    # The LDS layout moves operands around in LDS, not the order of the sums:
    # the unswizzled, 128-byte-line and 256-byte-line layouts must give the
    # same bits, and the library's layout must match the oracle.
    M, N, K = 1000, 1032, 200
    case = si.dense_case(M, N, K, 21, ab_dtype="bf16", with_c=True, c_dtype="bf16",
                         d_dtype="f32", scale=1.0 / np.sqrt(K))
    A, B, C = case.A.to(dev), case.B.to(dev), case.C.to(dev)
    say(f"layout variants {M}x{N}x{K}")
    outs = {swz: sg.gemm_layout(A, B, swz, C=C, out_dtype=torch.float32) for swz in (16, 8, 0)}
    torch.cuda.synchronize()
    ref, bound = oracle_dense(case)
    check_close(_np(outs[16]), ref, bound, "f32", "layout 16")
    assert torch.equal(outs[16], outs[8])
    assert torch.equal(outs[16], outs[0])


@pytest.mark.parametrize("with_c", [False, True])
def test_layout_io_variants_bit_identical(dev, with_c):
    # The input/output ablation on the library's 256x256 kernel: swizzled or
    # plain operand tiles x swizzled or plain C/D staging.  Layouts move
    # bytes in LDS, not the order of any sum: all four give the same bits,
    # and the library's combination matches the oracle.
    M, N, K = 4100, 4104, 192
    case = si.dense_case(M, N, K, 23, ab_dtype="bf16", with_c=with_c, c_dtype="bf16",
                         d_dtype="bf16", scale=1.0 / np.sqrt(K))
    A, B = case.A.to(dev), case.B.to(dev)
    C = case.C.to(dev) if with_c else None
    say(f"layout io variants {M}x{N}x{K} C={with_c}")
    outs = {}
    for ops in (16, 0):
        for out in (1, 0):
            outs[ops, out] = sg.gemm_layout_io(A, B, ops, out, C=C, out_dtype=torch.bfloat16)
            torch.cuda.synchronize()
            name = sg.gemm_last_kernel()
            assert name.startswith(f"pingpong16_gemm_kernel<bf16,k,k,swz{ops}"), name
            assert ("out_swz0" in name) == (out == 0), name
    ref, bound = oracle_dense(case)
    check_close(_np(outs[16, 1]), ref, bound, "bf16", "layout io 16/1")
    for key, d in outs.items():
        assert torch.equal(d, outs[16, 1]), key
    # the library's own call runs the swizzled/swizzled kernel
    d = sg.gemm(A, B, C=C, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(d, outs[16, 1])


def test_layout128_variants_bit_identical(dev):
    # The 128x128 kernel with the swizzles, no layout change and the padded
    # rows: same bits, and the library's layout matches the oracle.
    M, N, K = 1000, 1032, 200
    case = si.dense_case(M, N, K, 22, ab_dtype="bf16", with_c=True, c_dtype="bf16",
                         d_dtype="f32", scale=1.0 / np.sqrt(K))
    A, B, C = case.A.to(dev), case.B.to(dev), case.C.to(dev)
    say(f"layout128 variants {M}x{N}x{K}")
    outs = {lay: sg.gemm_layout128(A, B, lay, C=C, out_dtype=torch.float32)
            for lay in (16, 8, 0, sg.SG_LAYOUT_PAD16)}
    torch.cuda.synchronize()
    ref, bound = oracle_dense(case)
    check_close(_np(outs[16]), ref, bound, "f32", "layout128 16")
    for lay in (8, 0, sg.SG_LAYOUT_PAD16):
        assert torch.equal(outs[16], outs[lay]), lay


def test_dense_integer_inputs_exact(dev):
    # Integer values in [-4, 4]: every partial sum is exact in fp32, so the
    # result must be bit-exact whatever the summation order.
    M, N, K = 520, 392, 648
    a = si.integer_valued((M, K), 91)
    b = si.integer_valued((N, K), 92)
    A, B = si.to_bf16(a), si.to_bf16(b)
    say("integer-valued exact")
    d = sg.gemm(A.to(dev), B.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


def test_dense_256_tiles_integer_inputs_exact(dev):
    # The same on the 256x256 variant (17 x 17 tiles, ragged M and N): every
    # partial sum of values in [-4, 4] over K = 256 is exact in fp32.
    M, N, K = 4100, 4104, 256
    a = si.integer_valued((M, K), 93)
    b = si.integer_valued((N, K), 94)
    A, B = si.to_bf16(a), si.to_bf16(b)
    say(f"integer-valued exact, 256 tiles {M}x{N}x{K}")
    d = sg.gemm(A.to(dev), B.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


def test_gemm_plan_matches_gemm_and_oracle(dev):
    # The prepared call launches the same kernel with the same arguments:
    # bit-identical to gemm(), on the 1024^3 workload's shape family (64x64
    # tiles, B [K][N]), called twice.
    case = si.dense_case(200, 136, 264, 17, ab_dtype="bf16", a_major="k", b_major="mn",
                         with_c=True, c_dtype="bf16", d_dtype="f32")
    A, B, C = case.A.to(dev), case.B.to(dev), case.C.to(dev)
    say("gemm_plan vs gemm")
    want = sg.gemm(A, B, a_major="k", b_major="mn", C=C, out_dtype=torch.float32)
    out = torch.full_like(want, float("nan"))
    run = sg.gemm_plan(A, B, a_major="k", b_major="mn", C=C, out=out)
    run()
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    out.fill_(float("nan"))
    run()
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    ref, bound = oracle_dense(case)
    check_close(_np(out), ref, bound, "f32", "gemm_plan")


def test_dense_in_place_c_equals_d(dev):
    case = si.dense_case(128, 128, 96, 5, ab_dtype="bf16", with_c=True, c_dtype="f32",
                         d_dtype="f32")
    say("in-place C == D")
    CD = case.C.to(dev).clone()
    sg.gemm(case.A.to(dev), case.B.to(dev), C=CD, out=CD)
    torch.cuda.synchronize()
    ref, bound = oracle_dense(case)
    check_close(_np(CD), ref, bound, "f32", "in-place")


@pytest.mark.parametrize("a_major,b_major", [("k", "mn"), ("mn", "k"), ("mn", "mn")])
@pytest.mark.parametrize("K", [128, 320, 1024])
def test_dense_256_tiles_mn_major_integer_exact(dev, a_major, b_major, K):
    # A stored [K][M] and/or B stored [K][N] on 256x256 tiles: the ping-pong
    # keeps such an operand one 256-byte LDS row per k and reads fragments
    # with transposing reads.  Ragged M and N (8 rows and columns in the last
    # tiles: MN-major rows need a multiple of 8 elements); two, five and
    # sixteen K tiles.
    M, N = 4104, 4104
    a = si.integer_valued((M, K), 131 + K)
    b = si.integer_valued((N, K), 132 + K)
    A = si.to_bf16(a) if a_major == "k" else si.to_bf16(a).t().contiguous()
    B = si.to_bf16(b) if b_major == "k" else si.to_bf16(b).t().contiguous()
    say(f"integer-valued exact, 256 tiles, {a_major}/{b_major} {M}x{N}x{K}")
    d = sg.gemm(A.to(dev), B.to(dev), a_major=a_major, b_major=b_major,
                out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


def test_dense_256_tiles_mn_major_with_c(dev):
    # Both operands MN-major with a bf16 C brought in by the last loads and
    # bf16 D.
    M, N, K = 4104, 4104, 192
    case = si.dense_case(M, N, K, 133, ab_dtype="bf16", a_major="mn", b_major="mn",
                         with_c=True, c_dtype="bf16", d_dtype="bf16", scale=1.0 / np.sqrt(K))
    say(f"256 tiles, MN-major B, bf16 C {M}x{N}x{K}")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "bf16", "256 tiles MN-major B")


def test_dense_256_tiles_in_place_bf16(dev):
    # C == D on the 256x256 kernel with a bf16 C: each wave's C block comes
    # into LDS with the last K tiles' loads, before any of its D is written.
    M, N, K = 4100, 4104, 192
    case = si.dense_case(M, N, K, 21, ab_dtype="bf16", with_c=True, c_dtype="bf16",
                         d_dtype="bf16", scale=1.0 / np.sqrt(K))
    say("in-place C == D, 256 tiles, bf16")
    CD = case.C.to(dev).clone()
    sg.gemm(case.A.to(dev), case.B.to(dev), C=CD, out=CD)
    torch.cuda.synchronize()
    ref, bound = oracle_dense(case)
    check_close(_np(CD), ref, bound, "bf16", "in-place 256")


def test_dense_degenerate_shapes(dev):
    say("degenerate shapes")
    # K = 0: D = C exactly; and D = 0 without C.
    C = torch.randn(40, 64, device=dev)
    A = torch.empty(40, 0, dtype=torch.bfloat16, device=dev)
    B = torch.empty(64, 0, dtype=torch.bfloat16, device=dev)
    d = sg.gemm(A, B, C=C, out_dtype=torch.float32)
    d0 = sg.gemm(A, B, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(d, C) and torch.count_nonzero(d0) == 0
    # M = 0 and N = 0 leave D untouched.
    D = torch.full((8, 8), 7.0, device=dev)
    Bk = torch.zeros(8, 8, dtype=torch.bfloat16, device=dev)
    rc = sg.gemm_run(0, 8, 8, None, 0, Bk.data_ptr(), 0, sg.SG_BF16, None, 0,
                     D.data_ptr(), sg.SG_F32, None)
    torch.cuda.synchronize()
    assert rc == 0 and torch.all(D == 7.0)
    # Smallest legal rows: M = 1, N = 8 (bf16 out), K = 8.
    case = si.dense_case(1, 8, 8, 3, ab_dtype="bf16", d_dtype="bf16")
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "bf16", "1x8x8")


@pytest.mark.parametrize("K", [0, 8, 64])
@pytest.mark.parametrize("with_c", [False, True])
def test_dense_256_tiles_16bit_d_short_k(dev, K, with_c):
    # The 256x256 kernel writes a 16-bit D through LDS after any mainloop:
    # none (K = 0: D = C exactly, or zero), one partial K tile, one whole K
    # tile (a C is then read by the epilogue, not by the last loads).  N =
    # 4104 leaves 8 columns in the last tile column.
    M, N = 4096, 4104
    say(f"256 tiles, bf16 D through LDS, K={K} C={with_c}")
    if K == 0:
        g = torch.Generator().manual_seed(5)
        C = torch.randn(M, N, generator=g).to(torch.bfloat16).to(dev) if with_c else None
        A = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
        B = torch.empty(N, 0, dtype=torch.bfloat16, device=dev)
        d = sg.gemm(A, B, C=C, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(d, C) if with_c else torch.count_nonzero(d) == 0
        return
    case = si.dense_case(M, N, K, 60 + K, ab_dtype="bf16", with_c=with_c, c_dtype="bf16",
                         d_dtype="bf16", scale=1.0 / np.sqrt(K))
    d = run_dense(case, dev)
    ref, bound = oracle_dense(case)
    check_close(_np(d), ref, bound, "bf16", f"256 tiles K={K}")


def test_dense_8192_full_size(dev):
    # The headline workload in the bench's launch configuration, every one
    # of its 67,108,864 outputs against the oracle (all host cores, about
    # 20-40 s).
    case = si.dense_8192(seed=3)
    say(f"{case.name} (every output)")
    d = run_dense(case, dev)
    assert sg.gemm_last_kernel().startswith("pingpong16_gemm_kernel<bf16,k,k")
    got = _np(d)
    del d
    ref, bound = oracle_dense(case)
    check_close(got, ref, bound, "bf16", case.name)


# ------------------------------------------------------------- grouped

def test_grouped_small_with_empty_groups(dev):
    m_sizes = [0, 37, 128, 0, 300, 1, 256]
    case = si.grouped_case(m_sizes, 264, 200, 8, d_dtype="f32")
    say(f"grouped small {m_sizes}")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    check_close(_np(d), ref, bound, "f32", "grouped small")


@pytest.mark.parametrize("K", [200, 256])
def test_grouped_256_tiles_ragged(dev, K):
    # Enough tiles for the 256x256 variant; group sizes off the tile grid, an
    # empty group, and K = 3 * 64 + 8 (per-load K checks) or 4 * 64.
    m_sizes = [300, 1, 0, 777, 2000, 513, 1200]
    case = si.grouped_case(m_sizes, 4096, K, 13, d_dtype="f32")
    say(f"grouped 256-tile path {m_sizes} x 4096 x {K}")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    check_close(_np(d), ref, bound, "f32", "grouped 256 tiles")


def test_grouped_single_group_equals_dense(dev):
    case = si.grouped_case([300], 136, 72, 9, d_dtype="f32")
    say("grouped G=1 vs dense")
    A, B = case.A.to(dev), case.B.to(dev)
    dg = sg.grouped_gemm(A, B, case.m_offsets, out_dtype=torch.float32)
    dd = sg.gemm(A, B[0], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dg, dd)


def test_grouped_full_size(dev):
    # The grouped workload (16 groups x 4096 x 4096), every output.
    case = si.grouped(seed=4)
    say(f"{case.name} m_sizes={case.m_sizes} (every output)")
    d = sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets,
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("pingpong16_grouped_kernel<bf16")
    got = _np(d)
    del d
    ref, bound = oracle.grouped_gemm(case.m_offsets, case.N, case.K, case.A, case.B, "bf16")
    for g in range(case.G):
        lo, hi = case.m_offsets[g], case.m_offsets[g + 1]
        check_close(got[lo:hi], ref[lo:hi], bound[lo:hi], "bf16", f"group {g}")


# ------------------------------------------------------------------ MX

def run_mx_blocks(case: si.MXCase, dev, d_dtype="bf16"):
    """The case through mx_scales_to_blocks and mx_gemm_blocks_run."""
    sfa = sg.mx_scales_blocks(case.SFA.to(dev))
    sfb = sg.mx_scales_blocks(case.SFB.to(dev))
    d = sg.mx_gemm_blocks(case.A.to(dev), sfa, case.B.to(dev), sfb, fmt=case.fmt,
                          out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    return d


def blocks_reference(sf: np.ndarray) -> np.ndarray:
    """The SG_SF_BLOCKS image of e8m0 scales [rows][K/32], written out from
    its definition: byte b of row r at ((r // 64) * G + b // 16) * 1024 +
    (r % 64) * 16 + 8 * (b % 2) + (b % 16) // 2, G = ceil(K/512), zeros
    elsewhere."""
    rows, nb = sf.shape
    G = (nb + 15) // 16
    out = np.zeros(((rows + 63) // 64) * G * 1024, np.uint8)
    for r in range(rows):
        for b in range(nb):
            out[((r // 64) * G + b // 16) * 1024 + (r % 64) * 16 + 8 * (b % 2)
                + (b % 16) // 2] = sf[r, b]
    return out


@pytest.mark.parametrize("rows,K", [(1, 128), (100, 640), (300, 1024), (64, 512)])
def test_mx_scales_to_blocks_is_the_documented_permutation(dev, rows, K):
    rng = np.random.default_rng(rows + K)
    sf = rng.integers(0, 256, (rows, K // 32)).astype(np.uint8)
    say(f"mx_scales_to_blocks {rows}x{K // 32}")
    dst = torch.full((sg.mx_scales_blocks_bytes(rows, K),), 0xA5, dtype=torch.uint8,
                     device=dev)
    got = sg.mx_scales_blocks(torch.from_numpy(sf).to(dev), out=dst)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), blocks_reference(sf))


@pytest.mark.parametrize("fmt,M,N,K", [
    ("e4m3", 300, 264, 640), ("e4m3", 4100, 4104, 640), ("e4m3", 128, 128, 128),
    ("e2m1", 300, 264, 768), ("e2m1", 4100, 4104, 512),
    ("e2m3", 257, 36, 640), ("e3m2", 4100, 4104, 384), ("e2m3", 1, 4, 128),
])
def test_mx_blocks_scales_give_the_same_d(dev, fmt, M, N, K):
    # The same GEMM with the scales in the blocks layout: D bit-identical to
    # the rows layout's (which the tests above compare with the oracle), on
    # 128- and 256-wide tiles, ragged M and N, K not a multiple of 512 (a
    # partial last scale group) and scales over 2^-17 .. 2^17.
    case = si.mx_case(M, N, K, 31, fmt=fmt)
    rng = np.random.default_rng(9)
    case.SFA = torch.from_numpy(rng.integers(110, 145, (M, K // 32)).astype(np.uint8))
    case.SFB = torch.from_numpy(rng.integers(110, 145, (N, K // 32)).astype(np.uint8))
    say(f"mx blocks {fmt} {M}x{N}x{K}")
    runner = {"e4m3": run_mx, "e2m1": run_mx4, "e2m3": run_mx6, "e3m2": run_mx6}[fmt]
    for dt in ("f32", "bf16") if N % 8 == 0 else ("f32",):  # D rows of 16-byte multiples
        ref = runner(case, dev, dt)
        assert torch.equal(run_mx_blocks(case, dev, dt), ref), (fmt, dt)


def blocks_padding_mask(rows: int, K: int) -> np.ndarray:
    """The bytes of an SG_SF_BLOCKS array that hold no scale: rows past
    `rows` in the last 64-row block and blocks past K/32 in the last group."""
    used = blocks_reference(np.ones((rows, K // 32), np.uint8))
    return used == 0


@pytest.mark.parametrize("fmt,M,N,K", [
    ("e4m3", 300, 264, 640), ("e4m3", 100, 72, 384), ("e2m1", 300, 264, 768),
    ("e2m3", 257, 40, 640), ("e3m2", 260, 200, 384),
])
def test_mx_blocks_padding_is_never_used(dev, fmt, M, N, K):
    # The block layout pads rows to a multiple of 64 and blocks to a multiple
    # of 16; a caller that builds the array itself may leave anything there.
    # With every padding byte 255 (NaN scales) D stays bit-identical to the
    # zero-padded array's, on 128- and 256-wide tiles.
    case = si.mx_case(M, N, K, 41, fmt=fmt)
    say(f"mx blocks padding {fmt} {M}x{N}x{K}")
    sfa = sg.mx_scales_blocks(case.SFA.to(dev))
    sfb = sg.mx_scales_blocks(case.SFB.to(dev))
    A, B = case.A.to(dev), case.B.to(dev)
    ref = sg.mx_gemm_blocks(A, sfa, B, sfb, fmt=case.fmt, out_dtype=torch.float32)
    pa = torch.from_numpy(blocks_padding_mask(M, K)).to(dev)
    pb = torch.from_numpy(blocks_padding_mask(N, K)).to(dev)
    assert pa.any() and pb.any()
    sfa[pa] = 255
    sfb[pb] = 255
    got = sg.mx_gemm_blocks(A, sfa, B, sfb, fmt=case.fmt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref), fmt


def run_mx(case: si.MXCase, dev, d_dtype="bf16"):
    d = sg.mx_gemm(case.A.to(dev), case.SFA.to(dev), case.B.to(dev), case.SFB.to(dev),
                   out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (128, 128, 128), (520, 136, 256)])
def test_mx_small_full(dev, M, N, K):
    case = si.mx_case(M, N, K, 17)
    say(f"mx {M}x{N}x{K}")
    d = run_mx(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB)
    check_close(_np(d), ref, bound, "f32", "mx small", tau=tau_mx_f32(K))


def test_mx_scales_wide_range_and_unit(dev):
    M, N, K = 256, 264, 512
    case = si.mx_case(M, N, K, 18)
    rng = np.random.default_rng(5)
    case.SFA = torch.from_numpy(rng.integers(110, 145, (M, K // 32)).astype(np.uint8))
    case.SFB = torch.from_numpy(rng.integers(110, 145, (N, K // 32)).astype(np.uint8))
    say("mx wide scales")
    d = run_mx(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB)
    check_close(_np(d), ref, bound, "f32", "mx wide scales", tau=tau_mx_f32(K))
    case.SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    case.SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    d = run_mx(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB)
    check_close(_np(d), ref, bound, "f32", "mx unit scales", tau=tau_mx_f32(K))


def test_mx_256_tiles_ragged(dev):
    # 17 x 17 tiles of 256 (the 256x256 variant), ragged M and N, an odd
    # number of 128-wide K tiles, scales spread over 2^-17 .. 2^17.
    M, N, K = 4100, 4104, 384
    case = si.mx_case(M, N, K, 19)
    rng = np.random.default_rng(6)
    case.SFA = torch.from_numpy(rng.integers(110, 145, (M, K // 32)).astype(np.uint8))
    case.SFB = torch.from_numpy(rng.integers(110, 145, (N, K // 32)).astype(np.uint8))
    say(f"mx 256-tile path {M}x{N}x{K}")
    d = run_mx(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB)
    check_close(_np(d), ref, bound, "f32", "mx 256 tiles", tau=tau_mx_f32(K))


def run_mx4(case: si.MXCase, dev, d_dtype="bf16"):
    d = sg.mxfp4_gemm(case.A.to(dev), case.SFA.to(dev), case.B.to(dev), case.SFB.to(dev),
                      out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (4100, 4104, 768)])
def test_mxfp4_ragged(dev, M, N, K):
    # e2m1 elements; ragged M and N, an odd number of 256-wide K tiles in the
    # second case, scales spread over 2^-17 .. 2^17.
    case = si.mx_case(M, N, K, 23, fmt="e2m1")
    rng = np.random.default_rng(7)
    case.SFA = torch.from_numpy(rng.integers(110, 145, (M, K // 32)).astype(np.uint8))
    case.SFB = torch.from_numpy(rng.integers(110, 145, (N, K // 32)).astype(np.uint8))
    say(f"mxfp4 {M}x{N}x{K}")
    d = run_mx4(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB, fmt="e2m1")
    check_close(_np(d), ref, bound, "f32", "mxfp4")


def test_mxfp4_unit_scales_exact(dev):
    # e2m1 values are multiples of 1/2 below 8 and the scales are 1: every
    # partial sum is exact in fp32, so the result must be bit-exact.
    M, N, K = 520, 392, 1024
    rng = np.random.default_rng(24)
    A = torch.from_numpy(rng.integers(0, 256, (M, K // 2)).astype(np.uint8))
    B = torch.from_numpy(rng.integers(0, 256, (N, K // 2)).astype(np.uint8))
    SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    case = si.MXCase(M, N, K, A, SFA, B, SFB, "f32", "mxfp4 exact", "e2m1")
    say("mxfp4 unit scales exact")
    d = run_mx4(case, dev, "f32")
    ref, _ = oracle.mx_gemm(M, N, K, A, SFA, B, SFB, fmt="e2m1")
    assert np.array_equal(_np(d), ref)


def test_mxfp4_8192_full_size_sampled(dev):
    case = si.mxfp4()
    say(f"{case.name} (sampled)")
    d = run_mx4(case, dev, "bf16")
    assert bool(torch.isfinite(d).all())
    assert torch.equal(run_mx_blocks(case, dev, "bf16"), d)
    rows, cols = sample_points(case.M, case.N, 3000, 56)
    ref, bound = oracle.mx_gemm_points(case.M, case.N, case.K, case.A, case.SFA, case.B,
                                       case.SFB, rows, cols, fmt="e2m1")
    got = _np(d[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)])
    check_close(got, ref, bound, "bf16", case.name)


def run_mx6(case: si.MXCase, dev, d_dtype="bf16"):
    d = sg.mxfp6_gemm(case.A.to(dev), case.SFA.to(dev), case.B.to(dev), case.SFB.to(dev),
                      fmt=case.fmt, out_dtype=DT[d_dtype])
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (4100, 4104, 768), (257, 36, 128),
                                   (31, 292, 256), (1, 4, 128)])
def test_mxfp6_ragged(dev, fmt, M, N, K):
    # 6-bit elements; ragged M and N with the operands' last rows at odd and
    # even positions of their 32-row blocks (the rows the kernel leaves
    # unshifted), one-tile and many-tile grids, scales over 2^-17 .. 2^17.
    case = si.mx_case(M, N, K, 27, fmt=fmt)
    rng = np.random.default_rng(8)
    case.SFA = torch.from_numpy(rng.integers(110, 145, (M, K // 32)).astype(np.uint8))
    case.SFB = torch.from_numpy(rng.integers(110, 145, (N, K // 32)).astype(np.uint8))
    say(f"mxfp6 {fmt} {M}x{N}x{K}")
    d = run_mx6(case, dev, "f32")
    ref, bound = oracle.mx_gemm(M, N, K, case.A, case.SFA, case.B, case.SFB, fmt=fmt)
    check_close(_np(d), ref, bound, "f32", f"mxfp6 {fmt}",
                tau=tau_mx_f32(K) if fmt == "e3m2" else None)


def _pack6(codes: np.ndarray) -> torch.Tensor:
    """Rows of 6-bit codes as the stream format: four codes in three bytes,
    code k at bits [6k, 6k+6), little endian."""
    q = codes.astype(np.uint32).reshape(codes.shape[0], -1, 4)
    w = q[:, :, 0] | (q[:, :, 1] << 6) | (q[:, :, 2] << 12) | (q[:, :, 3] << 18)
    b = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=2).astype(np.uint8)
    return torch.from_numpy(np.ascontiguousarray(b.reshape(codes.shape[0], -1)))


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_mxfp6_unit_scales_exact(dev, fmt):
    # Unit scales and codes whose products and partial sums are exact in
    # fp32 (e2m3: multiples of 1/8 below 8; e3m2: magnitudes below 2,
    # multiples of 1/16): the result must be bit-exact.
    M, N, K = 520, 392, 1024
    rng = np.random.default_rng(25)
    hi = 64 if fmt == "e2m3" else 16
    ca = rng.integers(0, hi, (M, K)) | (rng.integers(0, 2, (M, K)) << 5)
    cb = rng.integers(0, hi, (N, K)) | (rng.integers(0, 2, (N, K)) << 5)
    A, B = _pack6(ca & 63), _pack6(cb & 63)
    SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    case = si.MXCase(M, N, K, A, SFA, B, SFB, "f32", f"mxfp6 {fmt} exact", fmt)
    say(f"mxfp6 {fmt} unit scales exact")
    d = run_mx6(case, dev, "f32")
    ref, _ = oracle.mx_gemm(M, N, K, A, SFA, B, SFB, fmt=fmt)
    assert np.array_equal(_np(d), ref)


def test_mxfp6_k0_is_zero(dev):
    M, N = 300, 264
    out = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    e = torch.empty(0, dtype=torch.uint8, device=dev)
    rc = sg.mxfp6_gemm_run(sg.SG_E3M2, M, N, 0, e.data_ptr(), e.data_ptr(), e.data_ptr(),
                           e.data_ptr(), out.data_ptr(), sg.SG_F32,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and bool((out == 0).all())


def test_mxfp6_8192_full_size_sampled(dev):
    case = si.mxfp6()
    say(f"{case.name} (sampled)")
    d = run_mx6(case, dev, "bf16")
    assert bool(torch.isfinite(d).all())
    assert torch.equal(run_mx_blocks(case, dev, "bf16"), d)
    rows, cols = sample_points(case.M, case.N, 3000, 57)
    ref, bound = oracle.mx_gemm_points(case.M, case.N, case.K, case.A, case.SFA, case.B,
                                       case.SFB, rows, cols, fmt=case.fmt)
    got = _np(d[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)])
    check_close(got, ref, bound, "bf16", case.name)


def test_mx_8192_full_size(dev):
    # The MXFP8 workload, every output.
    case = si.mxfp8(seed=5)
    say(f"{case.name} (every output)")
    d = run_mx(case, dev, "bf16")
    assert sg.gemm_last_kernel().startswith("pingpong_mx_kernel<e4m3")
    assert torch.equal(run_mx_blocks(case, dev, "bf16"), d)
    got = _np(d)
    del d
    ref, bound = oracle.mx_gemm(case.M, case.N, case.K, case.A, case.SFA, case.B, case.SFB)
    check_close(got, ref, bound, "bf16", case.name)
