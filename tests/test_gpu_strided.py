"""GPU parity of gemm_strided_run: D = alpha*A*B + beta*C with padded rows
(leading dimensions above the logical widths), against the oracle's gemm_ex
on the same padded buffers.  Every padding element of A, B and C is NaN, so a
kernel that reads one produces NaN; D's padding holds a sentinel that must
survive.  Tolerance as in the other parity tests, on the bound
|alpha| sum|a*b| + |beta| |c|."""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_swizzled_amd as sg
import oracle
from tests._tol import check_close

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
SENTINEL = 12288.0  # exact in bf16, fp16 and fp32


def say(msg):
    print(f"[gpu-strided] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load()
    return torch.device("cuda:0")


def _padded(x: torch.Tensor, ld: int, fill: float) -> torch.Tensor:
    """[rows][ld] CPU buffer holding x in its first columns, fill elsewhere."""
    buf = torch.full((x.shape[0], ld), fill, dtype=x.dtype)
    buf[:, :x.shape[1]] = x
    return buf


def _operands(M, N, K, a_major, b_major, ab, seed, pads=(24, 8, 40, 56)):
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn(M, K, generator=g) / K ** 0.5).to(DT[ab])
    b = (torch.randn(N, K, generator=g) / K ** 0.5).to(DT[ab])
    c = torch.randn(M, N, generator=g).to(torch.bfloat16)
    A = a if a_major == "k" else a.t().contiguous()
    B = b if b_major == "k" else b.t().contiguous()
    # Row pitches must be multiples of 16 bytes: leading dimensions are
    # rounded up to multiples of 8 elements.
    ru8 = lambda x: (x + 7) // 8 * 8
    lda, ldb = ru8(A.shape[1] + pads[0]), ru8(B.shape[1] + pads[1])
    ldc, ldd = ru8(N + pads[2]), ru8(N + pads[3])
    return (_padded(A, lda, float("nan")), lda, _padded(B, ldb, float("nan")), ldb,
            _padded(c, ldc, float("nan")), ldc, ldd)


def _run(dev, M, N, K, a_major, b_major, ab, Abuf, lda, Bbuf, ldb, Cbuf, ldc, ldd, alpha,
         beta, d_dtype):
    Ad, Bd = Abuf.to(dev), Bbuf.to(dev)
    a_cols = K if a_major == "k" else M
    b_cols = K if b_major == "k" else N
    Cv = Cbuf.to(dev)[:, :N] if Cbuf is not None else None
    Dbuf = torch.full((M, ldd), SENTINEL, dtype=DT[d_dtype], device=dev)
    sg.gemm_strided(Ad[:, :a_cols], Bd[:, :b_cols], a_major=a_major, b_major=b_major, C=Cv,
                    alpha=alpha, beta=beta, out=Dbuf[:, :N])
    torch.cuda.synchronize()
    assert bool((Dbuf[:, N:] == SENTINEL).all()), "D padding was written"
    return Dbuf[:, :N]


@pytest.mark.parametrize("a_major,b_major,ab", [("k", "k", "bf16"), ("mn", "k", "bf16"),
                                                ("k", "mn", "f16"), ("mn", "mn", "bf16")])
@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (4100, 4104, 136), (4100, 4104, 192),
                                   (300, 252, 136), (4100, 4108, 192)])
def test_strided_scaled_parity(dev, a_major, b_major, ab, M, N, K):
    # 300 x 264: 128x128 tiles; 4100 x 4104: 256x256 tiles, K = 136 on the
    # ping-pong's checked loader (K-major operands) or the two-stage kernel
    # (MN-major ones), K = 192 on the ping-pong's loader for K a multiple of
    # 64 (MN-major operands through transposing reads).
    # N = 252 and 4108 leave 252 and 12 columns in the last tile column.
    Abuf, lda, Bbuf, ldb, Cbuf, ldc, ldd = _operands(M, N, K, a_major, b_major, ab, M + K)
    alpha, beta = 1.5, -0.75
    say(f"strided {M}x{N}x{K} {a_major}/{b_major} {ab} lda={lda} ldb={ldb} ldc={ldc} ldd={ldd}")
    d = _run(dev, M, N, K, a_major, b_major, ab, Abuf, lda, Bbuf, ldb, Cbuf, ldc, ldd, alpha,
             beta, "bf16")
    ref, bound = oracle.gemm_ex(M, N, K, alpha, Abuf, lda, a_major, Bbuf, ldb, b_major, ab,
                                beta, Cbuf, ldc, "bf16")
    check_close(d.float().cpu().numpy().astype(np.float64), ref, bound, "bf16", "strided")


def test_strided_scaled_integer_exact(dev):
    # Integers in [-4, 4], K = 256, alpha = 2, beta = -3: every product, sum
    # and scaling is exact in fp32, so D equals the int64 result exactly.
    M, N, K = 4100, 4104, 256
    rng = np.random.default_rng(31)
    a = rng.integers(-4, 5, (M, K))
    b = rng.integers(-4, 5, (N, K))
    c = rng.integers(-8, 9, (M, N))
    lda, ldb, ldc, ldd = K + 64, K + 8, N + 24, N + 8
    Abuf = _padded(torch.from_numpy(a).to(torch.bfloat16), lda, float("nan"))
    Bbuf = _padded(torch.from_numpy(b).to(torch.bfloat16), ldb, float("nan"))
    Cbuf = _padded(torch.from_numpy(c).to(torch.float32), ldc, float("nan"))
    say("strided integer exact alpha=2 beta=-3")
    d = _run(dev, M, N, K, "k", "k", "bf16", Abuf, lda, Bbuf, ldb, Cbuf, ldc, ldd, 2.0, -3.0,
             "f32")
    want = 2 * (a @ b.T) - 3 * c
    assert np.array_equal(d.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("K,c_dtype,d_dtype,alpha,beta", [
    (128, "bf16", "f32", 1.0, 1.0),    # two K tiles: both carry C, no steady state
    (192, "f16", "f32", 2.0, -3.0),
    (512, "bf16", "bf16", 1.0, 1.0),
    (256, "f16", "f16", 1.0, 0.5),
    (64, "bf16", "f32", 1.0, 1.0),     # one K tile: C is read by the epilogue
])
def test_256_tiles_16bit_c_integer_exact(dev, K, c_dtype, d_dtype, alpha, beta):
    # The 256x256 kernel brings a 16-bit C into LDS with the loads of its last
    # two K tiles.  Ragged M (the last tile row has 4 rows, so its second wave
    # group is idle) and N = 4108 (the last tile column has 12 columns, C rows
    # padded with NaN past N): integers in [-4, 4] and C in [-8, 8] keep every
    # sum and scaling exact in fp32, so D is the exact value rounded once.
    M, N = 4100, 4108
    rng = np.random.default_rng(K)
    a = rng.integers(-4, 5, (M, K))
    b = rng.integers(-4, 5, (N, K))
    c = rng.integers(-8, 9, (M, N))
    ldc, ldd = N + 20, N + 4   # 16-byte row pitches
    Abuf = torch.from_numpy(a).to(torch.bfloat16)
    Bbuf = torch.from_numpy(b).to(torch.bfloat16)
    Cbuf = _padded(torch.from_numpy(c).to(DT[c_dtype]), ldc, float("nan"))
    say(f"256 tiles, {c_dtype} C in LDS, {M}x{N}x{K} D={d_dtype} alpha={alpha} beta={beta}")
    d = _run(dev, M, N, K, "k", "k", "bf16", Abuf, K, Bbuf, K, Cbuf, ldc, ldd, alpha, beta,
             d_dtype)
    exact = alpha * (a.astype(np.float64) @ b.astype(np.float64).T) + beta * c
    want = torch.from_numpy(exact).to(torch.float32).to(DT[d_dtype])
    assert torch.equal(d.cpu(), want)


def test_alpha_zero_and_beta_zero_read_nothing(dev):
    M, N, K = 520, 392, 72
    nan_a = torch.full((M, K), float("nan"), dtype=torch.bfloat16)
    nan_b = torch.full((N, K), float("nan"), dtype=torch.bfloat16)
    c = torch.arange(M * N, dtype=torch.float32).reshape(M, N) % 97
    say("alpha = 0: D = beta * C, A and B are NaN")
    d = _run(dev, M, N, K, "k", "k", "bf16", nan_a, K, nan_b, K, c, N, N, 0.0, 0.5, "f32")
    assert torch.equal(d.cpu(), 0.5 * c)
    ones_a = torch.ones((M, K), dtype=torch.bfloat16)
    ones_b = torch.ones((N, K), dtype=torch.bfloat16)
    nan_c = torch.full((M, N), float("nan"), dtype=torch.float32)
    say("beta = 0: C is NaN and not read")
    d = _run(dev, M, N, K, "k", "k", "bf16", ones_a, K, ones_b, K, nan_c, N, N, -1.5, 0.0,
             "f32")
    assert bool((d.cpu() == -1.5 * K).all())


@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (4100, 4104, 192)])
def test_unit_scales_packed_equal_gemm_run(dev, M, N, K):
    # alpha = beta = 1 with packed leading dimensions is gemm_run, bit for bit.
    g = torch.Generator().manual_seed(K)
    A = (torch.randn(M, K, generator=g) / K ** 0.5).to(torch.bfloat16).to(dev)
    B = (torch.randn(N, K, generator=g) / K ** 0.5).to(torch.bfloat16).to(dev)
    C = torch.randn(M, N, generator=g).to(torch.bfloat16).to(dev)
    say(f"unit scales vs gemm_run {M}x{N}x{K}")
    d1 = sg.gemm_strided(A, B, C=C, out_dtype=torch.bfloat16)
    d2 = sg.gemm(A, B, C=C, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)
