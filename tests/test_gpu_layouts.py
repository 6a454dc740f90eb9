"""GPU: the layouts on the hot path, byte for byte.

* LDS images.  gemm_lds_image_tile runs one loader of the 256x256 kernels
  once -- the 16-bit ping-pong's K-major halves (both loaders), its MN-major
  256-byte rows, the MXFP6 shifted rows and the C block of the epilogue --
  and dumps the LDS it filled.  Each image must hold every loaded byte at
  the place the oracle's restatement of that map gives (and the library's
  exported map, where there is one): the store into the swizzled tile and
  the read out of it use one map ("Swizzling explained properly", section
  "Sample swizzled matmul").
* The scaled MFMA's operand layout and arithmetic.  gemm_mfma_scale_probe
  runs one v_mfma_scale_f32_32x32x64_f8f6f4 on operands built from a logical
  32 x 64 block per the layouts the MX kernels rely on (which lane and byte
  feed which row, K element and 32-element block, which lane's scale byte
  scales which block, and where the accumulator lands), against the
  oracle's decode of the same codes.  The order of K inside one group of
  eight K elements cannot change the result and is not observable;
  everything else is.  The instruction does not add a block's products
  exactly: it adds each group of eight at a fixed point 13 bits below the
  group's largest exponent sum, truncating toward zero (measured; pinned
  here by cases whose sums are exact in fp32), which bounds how far an MX
  GEMM may differ from the exact blockwise sum the oracle computes.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_swizzled_amd as sg
import oracle
from oracle import swizzle

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-layouts] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load()
    return torch.device("cuda:0")


def _image(dev, kind, X: np.ndarray, row0, byte0, size=16384):
    rows, row_bytes = X.shape
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
    out = torch.full((size,), 0xA5, dtype=torch.uint8, device=dev)
    rc = sg.gemm_lds_image_tile(kind, Xd.data_ptr(), rows, row_bytes, row0, byte0,
                                out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.gemm_last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _window(X, r0, nr, b0, nb):
    """X[r0:r0+nr, b0:b0+nb] with zeros past the operand."""
    t = np.zeros((nr, nb), dtype=np.uint8)
    r1, b1 = min(X.shape[0], r0 + nr), min(X.shape[1], b0 + nb)
    if r1 > r0 and b1 > b0:
        t[:r1 - r0, :b1 - b0] = X[r0:r1, b0:b1]
    return t


# -------------------------------------------------- K-major halves (16-bit)

@pytest.mark.parametrize("kind", [sg.SG_IMG_HALF, sg.SG_IMG_HALF_KEXACT])
@pytest.mark.parametrize("rows,row_bytes,row0,byte0", [
    (512, 512, 128, 256),    # interior half (K = 256)
    (300, 384, 256, 128),    # 44 valid rows
    (300, 272, 128, 256),    # K = 136: a 16-byte K tail (checked loader only)
])
def test_pingpong_half_image(dev, kind, rows, row_bytes, row0, byte0):
    if kind == sg.SG_IMG_HALF_KEXACT and row_bytes % 128:
        pytest.skip("the K-exact loader serves K a multiple of 64 only")
    say(f"half image kind={kind} {rows}x{row_bytes} at ({row0},{byte0})")
    X = np.random.default_rng(rows + row_bytes + kind).integers(0, 256, (rows, row_bytes),
                                                                 dtype=np.uint8)
    got = _image(dev, kind, X, row0, byte0)
    want = swizzle.lds_image(_window(X, row0, 128, byte0, 128), line_bytes=256)
    assert np.array_equal(got, want)
    # the library's exported map says the same
    m = sg.gemm_lds_layout(128, 128)
    assert np.array_equal(m, swizzle.lds_tile_map(128, 128, 256))


# ------------------------------------------- MN-major 256-byte rows (16-bit)

@pytest.mark.parametrize("K,cols,row0,byte0", [
    (256, 512, 64, 256),     # interior: k rows 64..127, columns 128..255
    (100, 512, 64, 0),       # 36 valid k rows
    (192, 200, 0, 256),      # 72 valid columns (a 16-byte column tail)
])
def test_pingpong_mn256_image(dev, K, cols, row0, byte0):
    say(f"mn256 image K={K} cols={cols} at ({row0},{byte0})")
    X = np.random.default_rng(K + cols).integers(0, 256, (K, 2 * cols), dtype=np.uint8)
    got = _image(dev, sg.SG_IMG_MN256, X, row0, byte0)
    logical = _window(X, row0, 64, byte0, 256)
    want = np.zeros(16384, dtype=np.uint8)
    for k in range(64):
        for b in range(0, 256, 16):
            o = swizzle.mn256_offset(k, b)
            want[o:o + 16] = logical[k, b:b + 16]
    assert np.array_equal(got, want)


# -------------------------------------------------------- MXFP6 shifted rows

@pytest.mark.parametrize("rows,T,row0,t", [
    (600, 3, 256, 1),    # a tile below the operand's last: every odd row shifted
    (300, 2, 256, 0),    # the last tile: rows at block position 43 % 32 = 11 unshifted
    (287, 1, 256, 0),    # the last row at block position 30 (even): all odd rows shifted
])
def test_mxfp6_half_image(dev, rows, T, row0, t):
    row_bytes = 96 * T
    say(f"fp6 image {rows} rows x {row_bytes} bytes, tile at row {row0}, K tile {t}")
    X = np.random.default_rng(rows + T).integers(0, 256, (rows, row_bytes), dtype=np.uint8)
    got = _image(dev, sg.SG_IMG_FP6, X, row0, 96 * t)
    left = rows - row0
    u = 32 if left > 256 else (left - 1) % 32
    logical = _window(X, row0, 128, 96 * t, 96)
    lib_map = sg.gemm_lds_layout_mxfp6(128, u)
    for r in range(128):
        for q in range(12):
            o = swizzle.mxfp6_offset(r, 8 * q, u)
            assert o == lib_map[r, q]
            assert np.array_equal(got[o:o + 8], logical[r, 8 * q:8 * q + 8]), (r, q)


# ----------------------------------------------------------- the C block

@pytest.mark.parametrize("M,N,row0,n0", [
    (512, 768, 256, 256),   # interior tile
    (300, 264, 256, 256),   # 44 valid rows, 8 valid columns
])
def test_cblock_image(dev, M, N, row0, n0):
    say(f"cblock image C {M}x{N}, tile at ({row0},{n0})")
    X = np.random.default_rng(M + N).integers(0, 256, (M, 2 * N), dtype=np.uint8)
    got = _image(dev, sg.SG_IMG_CBLOCK, X, row0, 2 * n0, size=65536)
    lib_map = sg.gemm_lds_layout_cblock()
    rows_valid, cols_valid = min(128, M - row0), min(256, N - n0)
    for w in range(4):
        for r in range(128):
            for c in range(8):
                o = swizzle.cblock_offset(w, r, c)
                assert o == lib_map[w, r, c]
                col = 64 * w + 8 * c
                if r >= rows_valid:
                    assert not got[o:o + 16].any(), (w, r, c)   # rows past M: zero
                elif col < cols_valid:
                    src = X[row0 + r, 2 * (n0 + col):2 * (n0 + col) + 16]
                    assert np.array_equal(got[o:o + 16], src), (w, r, c)
                # columns past N are never read by the epilogue: not compared


# ------------------------------------------------- the scaled MFMA layout

# Per format: (MFMA format code, operand bytes a lane fills, decode name).
FMTS = {"e4m3": (0, 32), "e2m1": (4, 16), "e2m3": (2, 24), "e3m2": (3, 24)}


def _lane_bytes(fmt: str, codes: np.ndarray) -> np.ndarray:
    """[64][32] operand bytes of a 32-row x 64-k block of element codes, laid
    out as the MX kernels feed the MFMA: lane l = row (l % 32) + 32 h holds,
    for e4m3, K [16h, 16h+16) in bytes 0-15 and K [32+16h, 32+16h+16) in
    bytes 16-31; for e2m1, the 32 elements of block h in bytes 0-15, element
    2i in the low nibble of byte i; for e2m3/e3m2, the 32 elements of block h
    as a 6-bit stream in bytes 0-23."""
    out = np.zeros((64, 32), dtype=np.uint8)
    for l in range(64):
        row, h = l % 32, l // 32
        if fmt == "e4m3":
            out[l, :16] = codes[row, 16 * h:16 * h + 16]
            out[l, 16:] = codes[row, 32 + 16 * h:32 + 16 * h + 16]
        elif fmt == "e2m1":
            blk = codes[row, 32 * h:32 * h + 32].astype(np.uint8)
            out[l, :16] = blk[0::2] | (blk[1::2] << 4)
        else:
            blk = codes[row, 32 * h:32 * h + 32].astype(np.uint32).reshape(8, 4)
            w = blk[:, 0] | (blk[:, 1] << 6) | (blk[:, 2] << 12) | (blk[:, 3] << 18)
            out[l, :24] = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255],
                                   axis=1).reshape(-1).astype(np.uint8)
    return out


def _decode(fmt: str, codes: np.ndarray) -> np.ndarray:
    """fp64 values of element codes via the oracle's decoders."""
    if fmt == "e4m3":
        return oracle.decode("e4m3", codes.astype(np.uint8))
    if fmt == "e2m1":
        flat = codes.reshape(-1).astype(np.uint8)
        return oracle.decode("e2m1", flat[0::2] | (flat[1::2] << 4)).reshape(codes.shape)
    flat = codes.reshape(-1, 4).astype(np.uint32)
    w = flat[:, 0] | (flat[:, 1] << 6) | (flat[:, 2] << 12) | (flat[:, 3] << 18)
    packed = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=1).astype(np.uint8)
    return oracle.decode(fmt, packed.reshape(-1)).reshape(codes.shape)


def _probe(dev, fmt, a_bytes, b_bytes, sa, sb):
    code = FMTS[fmt][0]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    A, B, SA, SB = t(a_bytes), t(b_bytes), t(sa), t(sb)
    out = torch.zeros(64 * 16, dtype=torch.float32, device=dev)
    rc = sg.gemm_mfma_scale_probe(code, A.data_ptr(), B.data_ptr(), SA.data_ptr(),
                                  SB.data_ptr(), out.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.gemm_last_error()
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(64, 16).astype(np.float64)
    # Accumulator layout of the 32x32 MFMA: lane l, register r holds
    # D[i][j] with j = l % 32 (a row of the second operand) and i = 8 (r / 4)
    # + 4 (l / 32) + r % 4 (a row of the first).
    D = np.empty((32, 32))
    for l in range(64):
        for r in range(16):
            D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = o[l, r]
    return D


def _codes(fmt, rng, shape):
    if fmt == "e4m3":   # every code but the two NaNs (S.1111.111)
        c = rng.integers(0, 256, shape)
        return np.where((c & 0x7F) == 0x7F, 0x7E, c)
    return rng.integers(0, 16 if fmt == "e2m1" else 64, shape)


# Smallest exponent of each element format (that of its subnormals).
EMIN = {"e4m3": -6, "e3m2": -2, "e2m3": 0, "e2m1": 0}


def _group_truncated(fmt, va, vb, xa, xb):
    """The scaled MFMA's sum as measured on gfx950: the products of each
    group of 8 consecutive K elements are added at a fixed point whose last
    bit is 2^(e_max - 13), e_max the largest sum of the two operands'
    exponents in the group (an element's exponent: floor(log2 |x|), at least
    the format's smallest), each product truncated toward zero to it; group
    sums and scales then combine at fp32 precision.  Returns the fp64 value
    and the magnitude sum the fp32 combination's rounding is bounded by."""
    def ex(v):
        e = np.full(v.shape, EMIN[fmt], dtype=np.int64)
        nz = v != 0
        e[nz] = np.maximum(np.floor(np.log2(np.abs(v[nz]))).astype(np.int64), EMIN[fmt])
        return e
    ea, eb = ex(va), ex(vb)
    D = np.zeros((32, 32))
    mag = np.zeros((32, 32))
    for i in range(32):
        for j in range(32):
            p = va[i] * vb[j]
            es = np.where(p == 0, -10 ** 6, ea[i] + eb[j])
            for g in range(8):
                ks = slice(8 * g, 8 * g + 8)
                lsb = 2.0 ** (es[ks].max() - 13)
                t = (np.trunc(p[ks] / lsb) * lsb).sum() * xa[i, g // 4] * xb[j, g // 4]
                D[i, j] += t
                mag[i, j] += abs(t)
    return D, mag


@pytest.mark.parametrize("fmt", list(FMTS))
def test_scaled_mfma_operand_and_scale_layout(dev, fmt):
    say(f"scaled MFMA layout probe {fmt}")
    rng = np.random.default_rng(FMTS[fmt][0] + 71)
    ca, cb = _codes(fmt, rng, (32, 64)), _codes(fmt, rng, (32, 64))
    # a different scale for every (row, block), over 2^-6 .. 2^6
    sa = rng.integers(121, 134, 64).astype(np.uint8)
    sb = rng.integers(121, 134, 64).astype(np.uint8)
    ab, bb = _lane_bytes(fmt, ca), _lane_bytes(fmt, cb)
    used = FMTS[fmt][1]
    if used < 32:   # bytes the instruction does not read hold junk
        ab[:, used:] = rng.integers(0, 256, (64, 32 - used))
        bb[:, used:] = rng.integers(0, 256, (64, 32 - used))
    D = _probe(dev, fmt, ab, bb, sa, sb)
    va, vb = _decode(fmt, ca), _decode(fmt, cb)
    # the scale byte of lane (row + 32 b) scales block b of that row
    xa = np.exp2(sa.astype(np.float64) - 127).reshape(2, 32).T   # [row][block]
    xb = np.exp2(sb.astype(np.float64) - 127).reshape(2, 32).T
    want, mag = _group_truncated(fmt, va, vb, xa, xb)
    # eight group sums combined in fp32: at most 8 roundings of 2^-24 of
    # the magnitudes involved
    err = np.abs(D - want)
    assert np.all(err <= 8 * 2.0 ** -24 * mag), float((err / np.maximum(mag, 1e-300)).max())
    # and against the exact blockwise definition (what the oracle computes):
    # e2m1 and e2m3 lose nothing to the group alignment (their products span
    # less than 2^13), e3m2 and e4m3 may lose up to 7 * 2^-13 of a group's
    # magnitude
    exact = sum((va[:, 32 * b:32 * b + 32] @ vb[:, 32 * b:32 * b + 32].T)
                * np.outer(xa[:, b], xb[:, b]) for b in range(2))
    bound = sum((np.abs(va[:, 32 * b:32 * b + 32]) @ np.abs(vb[:, 32 * b:32 * b + 32]).T)
                * np.outer(xa[:, b], xb[:, b]) for b in range(2))
    tau = (8 * 2.0 ** -24) if fmt in ("e2m1", "e2m3") else (7 * 2.0 ** -13 + 8 * 2.0 ** -24)
    assert np.all(np.abs(D - exact) <= tau * bound)


def test_scaled_mfma_group_truncation_e4m3(dev):
    # Cases whose every sum is exact in fp32, so they show the group
    # alignment alone.  2^x codes: 2^8 = 0x78, 2^-5 = 0x10, 2^-6 = 0x08,
    # 2^-9 = 0x01, 1.0 = 0x38, 448 = 0x7E.
    say("scaled MFMA group truncation, e4m3")
    unit = np.full(64, 127, dtype=np.uint8)
    ca = np.zeros((32, 64), dtype=np.int64)
    cb = np.zeros((32, 64), dtype=np.int64)
    cb[0] = 0x38                                   # B row 0: all 1.0
    ca[0, 0], ca[0, 1] = 0x78, 0x10                # 256 + 2^-5: kept (13 bits below 2^8)
    ca[1, 0], ca[1, 1] = 0x78, 0x08                # 256 + 2^-6: dropped
    ca[2, 0], ca[2, 8] = 0x78, 0x01                # 256 + 2^-9 in the next group: kept
    ca[3, 0], ca[3, 1:32] = 0x7E, 0x08             # 448 + 31 * 2^-6: the 7 in its group dropped
    ca[4, 5], ca[4, 0:5], ca[4, 6:16] = 0x78, 0x08, 0x08   # a group is 8 aligned elements
    ca[5, 0], ca[5, 1] = 0x78, 0x91                # 256 - 1.125 * 2^-5: truncated toward zero
    ca[6, 32], ca[6, 33] = 0x78, 0x08              # the same in the second block
    ca[7, 0], ca[7, 1] = 0x38, 0x01                # 1 + 2^-9: kept (9 bits below)
    D = _probe(dev, "e4m3", _lane_bytes("e4m3", ca), _lane_bytes("e4m3", cb), unit, unit)
    want = [256 + 2.0 ** -5, 256.0, 256 + 2.0 ** -9, 448 + 24 * 2.0 ** -6,
            256 + 8 * 2.0 ** -6, 256 - 2.0 ** -5, 256.0, 1 + 2.0 ** -9]
    assert list(D[:8, 0]) == want
    # products are aligned on the sum of the operands' exponents: 448 * 448
    # (2^8 * 2^8 times 3.0625) keeps 2^3 and drops 2^2
    ca = np.zeros((32, 64), dtype=np.int64)
    ca[0, 0], ca[0, 1] = 0x7E, (3 + 7) << 3        # 448 * 448 + 2^3
    ca[1, 0], ca[1, 1] = 0x7E, (2 + 7) << 3        # 448 * 448 + 2^2
    cb = np.zeros((32, 64), dtype=np.int64)
    cb[0, 0], cb[0, 1] = 0x7E, 0x38
    D = _probe(dev, "e4m3", _lane_bytes("e4m3", ca), _lane_bytes("e4m3", cb), unit, unit)
    assert list(D[:2, 0]) == [200704.0 + 8, 200704.0]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scaled_mfma_block_membership_one_hot(dev, fmt):
    # One non-zero element per operand: the product is non-zero exactly when
    # both sit at the same (row pair, K element), and it is scaled by the
    # scale of the block the layout assigns that element to.
    say(f"scaled MFMA one-hot {fmt}")
    one = 0x38 if fmt == "e4m3" else 0x2   # 1.0 in e4m3 / e2m1
    rng = np.random.default_rng(9)
    sa = (127 + np.arange(64) % 7).astype(np.uint8)
    sb = (127 + (np.arange(64) // 32) * 3).astype(np.uint8)
    for _ in range(24):
        i, j, k = rng.integers(0, 32), rng.integers(0, 32), rng.integers(0, 64)
        k2 = k if rng.random() < 0.5 else (k + 1 + rng.integers(0, 63)) % 64
        ca = np.zeros((32, 64), dtype=np.int64)
        cb = np.zeros((32, 64), dtype=np.int64)
        ca[i, k] = one
        cb[j, k2] = one
        D = _probe(dev, fmt, _lane_bytes(fmt, ca), _lane_bytes(fmt, cb), sa, sb)
        want = np.zeros((32, 32))
        if k == k2:
            blk = k // 32
            want[i, j] = 2.0 ** (int(sa[i + 32 * blk]) - 127 + int(sb[j + 32 * blk]) - 127)
        assert np.array_equal(D, want), (i, j, k, k2)
