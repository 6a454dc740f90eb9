"""XOR swizzle maps -- oracle side (TEST INFRASTRUCTURE ONLY).

Written from the pages' definitions, independently of the HIP headers:

* ``xor_cell``: the swizzle f(r, c) = (r, c XOR r) on a grid of rows and
  columns ("Swizzling explained properly", section "What does swizzling
  do?").  With ``bits`` given only the low ``bits`` bits of the row take part,
  i.e. c XOR (r mod 2^bits) -- the bits-limited form the same page discusses
  for grids with more rows than columns (section "CUTLASS swizzling
  notation").
* ``swizzle_offset``: the same map written on byte offsets with the three
  parameters (bits, base, shift) of that page's CUTLASS notation: the
  ``bits``-wide field that starts at bit ``base`` (the column) is XORed with
  the field that starts at bit ``base + shift`` (the row); the low ``base``
  bits (the atom, 16 bytes when base = 4) never move.
* ``sw64_cell_address``: the SW64 K-major address of a 16-byte cell with its
  phase taken from the pattern start address ("LBO, SBO and SWZ for a
  tcgen05 tile", section 3).
* ``lds_tile_offset``: the map the gfx950 kernels use for a K-major operand
  tile in LDS.  Reading: "row" means the LDS bank-line index and "column"
  the 16-byte unit within the bank line, so the map is
  ``swizzle_offset(off, bits=u, base=4, shift=u)`` with 2^u = bank-line bytes
  / 16 (one 16-byte atom per unit, as on both the tcgen05 page and the
  swizzling page).
"""
from __future__ import annotations

import numpy as np

ATOM_BYTES = 16


def xor_cell(r: int, c: int, bits: int | None = None):
    """f(r, c) = (r, c XOR r), or (r, c XOR (r mod 2^bits))."""
    key = r if bits is None else r & ((1 << bits) - 1)
    return r, c ^ key


def swizzle_offset(offset: int, bits: int, base: int, shift: int) -> int:
    """Byte-offset XOR swizzle with parameters (bits, base, shift >= bits)."""
    if bits < 0 or base < 0 or shift < bits:
        raise ValueError("need bits >= 0, base >= 0 and shift >= bits")
    mask = (1 << bits) - 1
    row_field = (offset >> (base + shift)) & mask
    return offset ^ (row_field << base)


def sw64_cell_address(P: int, band: int, r: int, q: int, sbo: int = 512,
                      row_bytes: int = 64) -> int:
    """SW64 K-major cell address for an 8-row band of 64-byte rows.

    The XOR key advances every two 64-byte rows (one 128-byte line) and
    starts at the phase of the pattern start P, counted in 128-byte units
    modulo the 4-line period."""
    key = ((P >> 7) + (r >> 1)) & 3
    return P + band * sbo + row_bytes * r + ATOM_BYTES * (q ^ key)


def log2_exact(x: int) -> int:
    if x <= 0 or x & (x - 1):
        raise ValueError(f"{x} is not a power of two")
    return x.bit_length() - 1


def lds_tile_offset(row: int, chunk: int, row_bytes: int,
                    line_bytes: int) -> int:
    """Physical byte offset in an LDS stage of logical 16-byte chunk
    ``chunk`` of tile row ``row``, for a K-major tile with ``row_bytes`` per
    row and a bank line of ``line_bytes`` bytes."""
    u = log2_exact(line_bytes // ATOM_BYTES)
    return swizzle_offset(row * row_bytes + ATOM_BYTES * chunk, u, 4, u)


def lds_tile_map(rows: int, row_bytes: int, line_bytes: int) -> np.ndarray:
    """[rows][row_bytes/16] array of physical byte offsets."""
    chunks = row_bytes // ATOM_BYTES
    out = np.empty((rows, chunks), dtype=np.int64)
    for r in range(rows):
        for c in range(chunks):
            out[r, c] = lds_tile_offset(r, c, row_bytes, line_bytes)
    return out


def lds_image(tile: np.ndarray, line_bytes: int) -> np.ndarray:
    """Physical LDS bytes of a logical tile ``tile`` ([rows][row_bytes],
    uint8) stored under ``lds_tile_offset``."""
    t = np.ascontiguousarray(tile, dtype=np.uint8)
    rows, row_bytes = t.shape
    out = np.zeros(rows * row_bytes, dtype=np.uint8)
    m = lds_tile_map(rows, row_bytes, line_bytes)
    for r in range(rows):
        for c in range(row_bytes // ATOM_BYTES):
            o = int(m[r, c])
            out[o:o + ATOM_BYTES] = t[r, ATOM_BYTES * c:ATOM_BYTES * (c + 1)]
    return out


# ---------------------------------------------------------------------------
# The kernels' other LDS maps, restated from their definitions (the XOR of a
# unit index with a row key, as above), independently of the HIP headers.
# Each places whole units, so each is a bijection on its region; their bank
# behaviour is checked against the measured bank model elsewhere.
# ---------------------------------------------------------------------------

def mn256_offset(k: int, byte: int) -> int:
    """An MN-major half tile of the 16-bit 256x256 kernel: one 256-byte row
    per k; the 32-byte unit u of row k sits at unit u XOR key(k), with
    key(k) = (k mod 4) + 4 * (bit 3 of k)."""
    key = (k & 3) | (((k >> 3) & 1) << 2)
    return 256 * k + 32 * ((byte >> 5) ^ key) + (byte & 31)


def mxfp6_offset(row: int, byte: int, unshifted: int = 32) -> int:
    """Byte ``byte`` (< 96) of a 96-byte MXFP6 tile row in the 128-byte rows
    of the 256-byte-line XOR map, odd rows displaced by 8 bytes except those
    at block position ``unshifted`` (row mod 32; 32 for none)."""
    shift = 8 if (row & 1) and (row & 31) != unshifted else 0
    b = byte + shift
    return lds_tile_offset(row, b >> 4, 128, 256) + (b & 15)


def cblock_offset(w4: int, r: int, c: int) -> int:
    """Where 16-byte chunk ``c`` (< 8) of row ``r`` (< 128) of wave ``w4``'s
    128 x 64 block of a 16-bit C lives: quarter r // 32 (16 KiB each), the
    wave's 1 KiB region 4 * ((r // 8) mod 4) + w4, 128-byte row r mod 8, and
    chunk c XOR ((r // 2) mod 8)."""
    return ((r >> 5) * 16384 + (4 * ((r >> 3) & 3) + w4) * 1024 + (r & 7) * 128
            + 16 * (c ^ ((r >> 1) & 7)))
