"""Pins of the oracle's MXFP6 path (CPU only).

The e2m3 and e3m2 decodes are checked on all 64 codes against value sets
built as fixed-point multiples (not from the sign/exponent/fraction fields),
against the OCP FP6 extremes and against torch's e4m3 cast (every FP6 value
is an e4m3 value).  The 6-bit stream order is checked against a packer that
writes each code into a Python integer at bit 6k.  The GEMM is checked
against numpy on exact cases (unit scales; power-of-two block scales).  The
quantizer that makes the MXFP6 workload is checked for its scale rule and
rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

# Non-negative magnitudes in code order.  E2M3: 0..15 eighths (subnormals and
# the first binade share the 1/8 spacing), then 8..15 quarters, 8..15 halves.
E2M3 = [k / 8 for k in range(16)] + [k / 4 for k in range(8, 16)] + [k / 2 for k in range(8, 16)]
# E3M2: 0..7 sixteenths, then 4..7 times 1/8, 1/4, 1/2, 1, 2, 4.
E3M2 = [k / 16 for k in range(8)] + [k * s for s in (1 / 8, 1 / 4, 1 / 2, 1, 2, 4)
                                     for k in range(4, 8)]
TABLE = {"e2m3": E2M3, "e3m2": E3M2}
FMTS = ["e2m3", "e3m2"]


def _pack6(codes: np.ndarray) -> np.ndarray:
    """Pack rows of 6-bit codes: code k of a row at bits [6k, 6k+6) of a
    little-endian byte string (one Python integer per row)."""
    rows, n = codes.shape
    assert n % 4 == 0
    out = np.empty((rows, 3 * n // 4), dtype=np.uint8)
    for r in range(rows):
        v = 0
        for k, c in enumerate(codes[r].tolist()):
            v |= int(c) << (6 * k)
        out[r] = np.frombuffer(v.to_bytes(3 * n // 4, "little"), dtype=np.uint8)
    return out


def _values(fmt: str, codes: np.ndarray) -> np.ndarray:
    t = np.array(TABLE[fmt] + [-v for v in TABLE[fmt]])
    return t[codes]


def _unpack6(packed: torch.Tensor) -> np.ndarray:
    """Codes of a packed 6-bit stream, by reading bit 6k.. of each row."""
    p = packed.numpy()
    rows, nb = p.shape
    out = np.empty((rows, 4 * nb // 3), dtype=np.int64)
    for r in range(rows):
        v = int.from_bytes(p[r].tobytes(), "little")
        for k in range(out.shape[1]):
            out[r, k] = (v >> (6 * k)) & 63
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_all_codes_match_value_sets(fmt):
    codes = np.arange(64, dtype=np.int64)[None, :]
    ours = oracle.decode(fmt, _pack6(codes))
    assert ours.shape == (64,)
    assert ours[:32].tolist() == TABLE[fmt]
    assert ours[32:].tolist() == [-v for v in TABLE[fmt]]   # bit 5 is the sign
    assert len(set(TABLE[fmt])) == 32 and TABLE[fmt] == sorted(TABLE[fmt])
    # OCP FP6 extremes: largest normal, smallest subnormal
    top, tiny = {"e2m3": (7.5, 0.125), "e3m2": (28.0, 0.0625)}[fmt]
    assert ours[31] == top and ours[1] == tiny
    # exactly representable in e4m3 (torch's cast is a library routine)
    t = torch.tensor(ours).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(t, ours)


@pytest.mark.parametrize("fmt", FMTS)
def test_stream_order(fmt):
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 64, (3, 16))
    packed = _pack6(codes)
    ours = oracle.decode(fmt, packed).reshape(3, 16)
    assert np.array_equal(ours, _values(fmt, codes))
    # one element alone in each of the four bit phases of a 3-byte group
    for k in range(8):
        one = np.zeros((1, 8), dtype=np.int64)
        one[0, k] = 31
        d = oracle.decode(fmt, _pack6(one))
        assert np.flatnonzero(d).tolist() == [k] and d[k] == TABLE[fmt][31]


@pytest.mark.parametrize("fmt", FMTS)
def test_unit_scales_equal_plain_product(fmt):
    M, N, K = 6, 5, 128
    rng = np.random.default_rng(22)
    ca, cb = rng.integers(0, 64, (M, K)), rng.integers(0, 64, (N, K))
    A, B = torch.from_numpy(_pack6(ca)), torch.from_numpy(_pack6(cb))
    SFA = torch.full((M, K // 32), 127, dtype=torch.uint8)
    SFB = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ref, bound = oracle.mx_gemm(M, N, K, A, SFA, B, SFB, fmt=fmt)
    a, b = _values(fmt, ca), _values(fmt, cb)
    # values are multiples of 1/16 below 32: products and sums are exact
    assert np.array_equal(ref, a @ b.T)
    assert np.array_equal(bound, np.abs(a) @ np.abs(b).T)


@pytest.mark.parametrize("fmt", FMTS)
def test_integer_codes_match_int64(fmt):
    # codes whose values are integers: the product is an int64 matmul
    ints = [c for c, v in enumerate(TABLE[fmt]) if v == int(v)]
    M, N, K = 7, 9, 96
    rng = np.random.default_rng(23)
    ca = rng.choice(ints, (M, K)) | (rng.integers(0, 2, (M, K)) << 5)
    cb = rng.choice(ints, (N, K)) | (rng.integers(0, 2, (N, K)) << 5)
    SF = torch.full((max(M, N), K // 32), 127, dtype=torch.uint8)
    ref, _ = oracle.mx_gemm(M, N, K, torch.from_numpy(_pack6(ca)), SF[:M],
                            torch.from_numpy(_pack6(cb)), SF[:N], fmt=fmt)
    ia = _values(fmt, ca).astype(np.int64)
    ib = _values(fmt, cb).astype(np.int64)
    assert np.array_equal(ref, (ia @ ib.T).astype(np.float64))


@pytest.mark.parametrize("fmt", FMTS)
def test_each_scale_applies_to_its_own_block(fmt):
    M, N, K = 3, 4, 96
    rng = np.random.default_rng(24)
    ca, cb = rng.integers(0, 64, (M, K)), rng.integers(0, 64, (N, K))
    sa = rng.integers(118, 137, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    ref, _ = oracle.mx_gemm(M, N, K, torch.from_numpy(_pack6(ca)), torch.from_numpy(sa),
                            torch.from_numpy(_pack6(cb)), torch.from_numpy(sb), fmt=fmt)
    a, b = _values(fmt, ca), _values(fmt, cb)
    expect = np.zeros((M, N))
    for blk in range(K // 32):
        sl = slice(32 * blk, 32 * blk + 32)
        expect += (a[:, sl] @ b[:, sl].T) \
            * np.ldexp(1.0, sa[:, blk].astype(np.int64) - 127)[:, None] \
            * np.ldexp(1.0, sb[:, blk].astype(np.int64) - 127)[None, :]
    assert np.array_equal(ref, expect)


@pytest.mark.parametrize("fmt", FMTS)
def test_points_agree_with_full(fmt):
    case = si.mx_case(33, 20, 256, 25, fmt=fmt)
    assert case.A.shape == (33, 192) and case.B.shape == (20, 192)
    ref, bound = oracle.mx_gemm(case.M, case.N, case.K, case.A, case.SFA, case.B, case.SFB,
                                fmt=fmt)
    rows, cols = [0, 32, 7], [19, 0, 11]
    rp, bp = oracle.mx_gemm_points(case.M, case.N, case.K, case.A, case.SFA, case.B,
                                   case.SFB, rows, cols, fmt=fmt)
    assert np.array_equal(rp, ref[rows, cols]) and np.array_equal(bp, bound[rows, cols])


@pytest.mark.parametrize("fmt", FMTS)
def test_quantizer_scale_and_rounding(fmt):
    rng = np.random.default_rng(26)
    x = rng.standard_normal((5, 128)).astype(np.float32)
    x[1, 64:96] = 0.0
    packed, scales = si.mxfp6_quantize(x, fmt)
    assert packed.shape == (5, 96) and scales.shape == (5, 4)
    xb = x.reshape(5, 4, 32)
    amax = np.abs(xb).max(axis=2)
    X = np.ldexp(1.0, scales.numpy().astype(np.int64) - 127)
    nz = amax > 0
    lo = {"e2m3": 4.0, "e3m2": 16.0}[fmt]
    # the block's absmax lands in the top binade [lo X, 2 lo X)
    assert np.all(lo * X[nz] <= amax[nz]) and np.all(amax[nz] < 2 * lo * X[nz])
    assert X[1, 2] == 1.0
    dec = _values(fmt, _unpack6(packed)).reshape(5, 4, 32)
    y = xb / X[:, :, None]
    # nearest value: within half the gap to a neighbour in the sorted table
    t = np.array(TABLE[fmt])
    mag = np.minimum(np.abs(y), t[-1])
    err = np.abs(np.abs(dec) - mag)
    best = np.abs(t[None, :] - mag.reshape(-1, 1)).min(axis=1).reshape(mag.shape)
    assert np.all(err <= best + 1e-12)
    assert np.all((np.sign(dec) == np.sign(y)) | (dec == 0))


def test_quantizer_ties_go_to_even_code():
    # block absmax 4 -> X = 1 for e2m3; 1.0625 lies halfway between 1.0
    # (code 8) and 1.125 (code 9); 1.1875 between 1.125 (9) and 1.25 (10)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :4] = [4.0, 1.0625, 1.1875, -1.0625]
    packed, scales = si.mxfp6_quantize(x, "e2m3")
    assert scales.tolist() == [[127]]
    assert _unpack6(packed)[0, :4].tolist() == [24, 8, 10, 32 | 8]   # 4.0 is code 24
