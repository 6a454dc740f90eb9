"""Pins of the oracle's swizzle maps and bank simulator (CPU only).

Against: the worked examples printed on the pages (tests/golden/*.json, each
entry citing its page and section), the swizzle theorems (bijection; elements
of one row, and of one column, land in distinct columns), and the equality
of the byte-offset form with the (row, column) form.
"""
import json
import os

import numpy as np
import pytest

from oracle import banks, swizzle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------- page worked examples

def test_tcgen05_unswizzled_a_tile_bytes_and_banks():
    g = _gold("tcgen05_a_tile_sw64.json")
    ld = g["loader"]
    t = g["tile"]
    chunks = t["BK"] * t["elem_bytes"] // 16
    assert chunks == ld["chunks_per_row"]
    assert t["threads"] // chunks == ld["rows_per_iteration"]
    assert t["BM"] // (t["threads"] // chunks) == ld["iterations"]
    row_bytes = t["BK"] * t["elem_bytes"]
    for m, q, byte in g["unswizzled"]["byte_of_m_q"]:
        # Unswizzled: no XOR (bits = 0).
        assert swizzle.swizzle_offset(row_bytes * m + 16 * q, 0, 4, 0) == byte
    for q, (lo, hi) in enumerate(g["unswizzled"]["relative_banks_of_q"]):
        assert (16 * q // 4, (16 * q + 15) // 4) == (lo, hi)
    assert [row_bytes * m for m in range(8)] == g["unswizzled"]["q0_row_start_bytes"]


def test_tcgen05_sw64_banks_keys_and_phase():
    g = _gold("tcgen05_a_tile_sw64.json")["sw64"]
    for r, (lo, hi) in enumerate(g["q0_banks_by_row"]):
        a = swizzle.sw64_cell_address(0, 0, r, 0)
        assert ((a // 4) % 32, ((a + 15) // 4) % 32) == (lo, hi)
    for P, keys in ((0, g["keys_mbo0"]), (128, g["keys_pattern_start_128"])):
        got = [(swizzle.sw64_cell_address(P, 0, r, 0) - P - 64 * r) // 16 for r in range(8)]
        assert got == keys
    assert g["sbo_bytes"] == 8 * 64 and g["sbo_encoded"] == g["sbo_bytes"] // 16
    # SW64 on 64-byte rows is the byte-offset swizzle (2, 4, 3) on 128-byte
    # lines: the key advances once per two rows.
    for band in range(2):
        for r in range(8):
            for q in range(4):
                off = band * 512 + 64 * r + 16 * q
                assert swizzle.sw64_cell_address(0, band, r, q) == \
                    swizzle.swizzle_offset(off, 2, 4, 3)


def test_swizzle_modes_sw32_row1_and_periods():
    g = _gold("swizzle_modes_128B.json")
    m = g["modes"]["SW32"]
    row = 1
    after = []
    for pos in range(8):
        # The logical cell that lands at physical position `pos` of row 1.
        for c in range(8):
            off = swizzle.swizzle_offset(128 * row + 16 * c, m["bits"], m["base"], m["shift"])
            if off == 128 * row + 16 * pos:
                after.append(8 * row + c)
    assert after == g["sw32_row1_cells"]["after"]
    for name in ("SW32", "SW64", "SW128"):
        m = g["modes"][name]
        perms = [[swizzle.swizzle_offset(128 * r + 16 * c, m["bits"], 4, 3) - 128 * r
                  for c in range(8)] for r in range(16)]
        period = next(p for p in range(1, 17) if all(perms[r] == perms[r % p] for r in range(16)))
        assert period == m["period_rows"]


def test_functor_equals_cell_form():
    g = _gold("swizzle_modes_128B.json")["functor_example"]
    for r in range(g["rows"]):
        for c in range(g["cols"]):
            off = r * g["cols"] + c
            rr, cc = swizzle.xor_cell(r, c)
            assert swizzle.swizzle_offset(off, g["bits"], g["base"], g["shift"]) == \
                rr * g["cols"] + cc
    # With 16-byte atoms (base 4) the same holds cell by cell, bytes kept.
    for r in range(8):
        for c in range(8):
            for byte in (0, 5, 15):
                rr, cc = swizzle.xor_cell(r, c, bits=3)
                assert swizzle.swizzle_offset(128 * r + 16 * c + byte, 3, 4, 3) == \
                    128 * rr + 16 * cc + byte


# ------------------------------------------------------------ bank degrees

def _ldmatrix_addrs(bits):
    """Eight 16-byte row addresses of one 8x16B operand (column 0) in a
    128-byte-pitch tile; bits = None for no swizzle."""
    out = []
    for r in range(8):
        off = 128 * r
        out.append(off if bits is None else swizzle.swizzle_offset(off, bits, 4, 3))
    return out


def test_page_ldmatrix_degrees():
    g = _gold("swizzle_modes_128B.json")
    for name, bits in (("none", None), ("SW32", 1), ("SW64", 2), ("SW128", 3)):
        d = banks.conflict_degree(_ldmatrix_addrs(bits), 16, nbanks=32, lanes_per_phase=8)
        assert d == g["modes"][name]["ldmatrix_degree"], name
    rp = g["row_pitch_128_conflict"]
    assert banks.conflict_degree([rp["row_bytes"] * r for r in range(rp["rows"])], 16,
                                 nbanks=32, lanes_per_phase=8) == rp["degree"]


def test_page_store_transaction_split_halves_degree():
    g = _gold("swizzle_modes_128B.json")["store_phase_split"]
    # Fragment layout of the page's fp32 store: lane = 4*group + t writes two
    # floats of row `group` at column 2t.
    addrs = [(lane // 4) * g["row_bytes"] + (lane % 4) * g["lane_bytes"]
             for lane in range(g["lanes"])]
    one = banks.conflict_degree(addrs, g["lane_bytes"], nbanks=32, lanes_per_phase=32)
    two = banks.conflict_degree(addrs, g["lane_bytes"], nbanks=32, lanes_per_phase=16)
    assert (one, two) == (g["degree_one_phase"], g["degree_two_phases"])


def test_broadcast_and_extra_cycles():
    # Identical addresses are one word: no conflict.
    assert banks.conflict_degree([0] * 8, 4, nbanks=32, lanes_per_phase=8) == 1
    # Two phases of degree 8 and 1 -> 7 extra cycles.
    a = [128 * r for r in range(8)] + [16 * r for r in range(8)]
    assert banks.phase_degrees(a, 16, nbanks=32, lanes_per_phase=8) == [8, 1]
    assert banks.extra_cycles(a, 16, nbanks=32, lanes_per_phase=8) == 7


# -------------------------------------------- kernel map: theorem checks

@pytest.mark.parametrize("line_bytes", [128, 256])
@pytest.mark.parametrize("row_bytes,rows", [(128, 256), (64, 128), (256, 64)])
def test_lds_tile_map_is_bijection_and_keeps_atoms(line_bytes, row_bytes, rows):
    m = swizzle.lds_tile_map(rows, row_bytes, line_bytes)
    flat = np.sort(m.ravel())
    assert np.array_equal(flat, 16 * np.arange(rows * row_bytes // 16))
    # The map only permutes 16-byte units inside one bank line.
    logical = (np.arange(rows)[:, None] * row_bytes + 16 * np.arange(row_bytes // 16)[None, :])
    assert np.all(m // line_bytes == logical // line_bytes)


@pytest.mark.parametrize("line_bytes", [128, 256])
def test_lds_tile_map_row_and_column_distinctness(line_bytes):
    # Theorem 1 (same row -> distinct columns) and theorem 2 (same column ->
    # distinct columns) on the bank-line grid the map is defined on.
    units = line_bytes // 16
    lines = units  # one full period
    for L in range(lines):
        cols = [(swizzle.swizzle_offset(L * line_bytes + 16 * c, units.bit_length() - 1, 4,
                                        units.bit_length() - 1) % line_bytes) // 16
                for c in range(units)]
        assert sorted(cols) == list(range(units))
    for c in range(units):
        cols = [(swizzle.swizzle_offset(L * line_bytes + 16 * c, units.bit_length() - 1, 4,
                                        units.bit_length() - 1) % line_bytes) // 16
                for L in range(lines)]
        assert sorted(cols) == list(range(units))


def test_lds_image_roundtrip():
    rng = np.random.default_rng(0)
    tile = rng.integers(0, 256, (32, 128), dtype=np.uint8)
    img = swizzle.lds_image(tile, 256)
    m = swizzle.lds_tile_map(32, 128, 256)
    for r in range(32):
        for c in range(8):
            assert np.array_equal(img[m[r, c]:m[r, c] + 16], tile[r, 16 * c:16 * c + 16])


# ------------------------------------------------- the kernels' other maps

def test_mn256_offset_is_a_bijection_of_whole_units():
    offs = [swizzle.mn256_offset(k, b) for k in range(64) for b in range(256)]
    assert sorted(offs) == list(range(64 * 256))
    for k in range(64):                       # 32-byte units stay whole
        for u in range(8):
            base = swizzle.mn256_offset(k, 32 * u)
            assert base % 32 == 0
            assert [swizzle.mn256_offset(k, 32 * u + i) for i in range(32)] == \
                list(range(base, base + 32))


def test_mn256_rows_of_one_transposing_read_use_distinct_units():
    # A read covers rows k0..k0+3 and k0+8..k0+11 at one logical unit: the
    # keys must give those eight rows eight different physical units.
    for k0 in range(0, 64, 16):
        for rr in (0, 4):
            rows = [k0 + rr + d for d in (0, 1, 2, 3, 8, 9, 10, 11)]
            for u in range(8):
                units = {(swizzle.mn256_offset(k, 32 * u) % 256) // 32 for k in rows}
                assert len(units) == 8


@pytest.mark.parametrize("unshifted", [32, 0, 11, 31])
def test_mxfp6_offset_places_every_byte_once(unshifted):
    offs = [swizzle.mxfp6_offset(r, b, unshifted) for r in range(128) for b in range(96)]
    assert len(set(offs)) == len(offs)
    for r in range(128):
        # a row's bytes stay in the 256-byte bank line of its two-row pair
        # (the XOR moves units only within a line)
        lines = {o // 256 for o in (swizzle.mxfp6_offset(r, b, unshifted) for b in range(96))}
        assert lines == {r // 2}


def test_cblock_offset_is_a_bijection_of_the_four_quarters():
    offs = [swizzle.cblock_offset(w, r, c) for w in range(4) for r in range(128)
            for c in range(8)]
    assert sorted(offs) == list(range(0, 65536, 16))
