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
