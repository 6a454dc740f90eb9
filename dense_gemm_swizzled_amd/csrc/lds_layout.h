// lds_layout.h -- the LDS byte map of a K-major operand tile (host + device).
//
// The swizzle is f(r, c) = (r, c XOR r) of "Swizzling explained properly"
// (section "What does swizzling do?") taken on the grid whose rows are LDS
// bank lines and whose columns are the 16-byte units of a line.  In that
// page's byte-offset notation (section "CUTLASS swizzling notation") it is
// Swizzle(bits = u, base = 4, shift = u) with 2^u units per line: the low 4
// bits (one 16-byte atom -- the same atom as the "core matrix" rows of "LBO,
// SBO and SWZ for a tcgen05 tile", section 1) never move, and the unit index
// inside a line is XORed with the line index modulo 2^u.
//
// gfx950's LDS serves ds_read_b128 from 64 banks of 4 bytes, a 256-byte line
// (measured with the LDS probe: two lanes 256 bytes apart conflict, 128
// bytes apart do not), so the kernels use u = 4 (Swz = 16 units).  Swz = 8
// is the same construction for 128-byte lines (the tcgen05/TMA 128-byte mode)
// and Swz = 0 the unswizzled layout; both stay selectable for the layout
// ablation.  Stage bases are multiples of the 4 KiB swizzle period, so the
// map's phase is the same in every stage (the matrix-base-offset issue of
// "LBO, SBO and SWZ for a tcgen05 tile", section 3, cannot arise).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SG_HD __host__ __device__ __forceinline__
#else
#define SG_HD inline
#endif

namespace sg {

constexpr int kSwzDefault = 16;

// The padded layout of "Swizzling explained properly" (the alternative it
// weighs against the swizzle): no XOR, every row followed by 16 bytes of
// padding (a 144-byte row stride for 128-byte rows), so consecutive rows
// start 36 banks apart.  Selected by Swz = kSwzPad, for the layout ablation.
constexpr int kSwzPad = -1;

// Bytes from one tile row to the next.
template <int RowBytes, int Swz>
SG_HD constexpr uint32_t lds_row_stride() {
  return Swz == kSwzPad ? RowBytes + 16 : RowBytes;
}

// Byte offset, within one stage, of logical 16-byte chunk `chunk` of tile
// row `row`, for rows of RowBytes bytes and a line of Swz 16-byte units.
template <int RowBytes, int Swz>
SG_HD constexpr uint32_t lds_offset(uint32_t row, uint32_t chunk) {
  static_assert(Swz == 0 || Swz == 8 || Swz == 16 || Swz == kSwzPad, "unsupported layout");
  const uint32_t off = row * lds_row_stride<RowBytes, Swz>() + chunk * 16u;
  if constexpr (Swz == 0 || Swz == kSwzPad) {
    return off;
  } else {
    constexpr uint32_t line_shift = Swz == 8 ? 7 : 8;  // log2(line bytes)
    return off ^ (((off >> line_shift) & (uint32_t)(Swz - 1)) << 4);
  }
}

// The same XOR applied to a byte offset within a stage (it is its own
// inverse: the key bits, above bit 7 or 8, are left unchanged).
template <int Swz>
SG_HD constexpr uint32_t swz_bytes(uint32_t off) {
  static_assert(Swz != kSwzPad, "the padded layout is not a permutation of a stage");
  if constexpr (Swz == 0) {
    return off;
  } else {
    constexpr uint32_t line_shift = Swz == 8 ? 7 : 8;
    return off ^ (((off >> line_shift) & (uint32_t)(Swz - 1)) << 4);
  }
}

// Runtime-dispatched form for host tools.
SG_HD uint32_t lds_offset_rt(int row_bytes, int swz, uint32_t row,
                             uint32_t chunk) {
  if (swz == kSwzPad) return row * (uint32_t)(row_bytes + 16) + chunk * 16u;
  const uint32_t off = row * (uint32_t)row_bytes + chunk * 16u;
  if (swz == 0) return off;
  const uint32_t line_shift = swz == 8 ? 7 : 8;
  return off ^ (((off >> line_shift) & (uint32_t)(swz - 1)) << 4);
}

// The MXFP6 operand tile.  A K tile of a 6-bit operand row is 96 bytes (128
// values), kept in the 128-byte rows of lds_offset<128, kSwzDefault>.  The
// scaled MFMA takes a lane's 32 values as 24 bytes, so a fragment is read
// with three 8-byte reads, each serving 32 lanes (rows R..R+31 of one
// 32-row block, all at the same byte of the row) from the 64 banks at once.
// The XOR moves whole 16-byte units, so on its own it gives those 32 reads
// only 16 distinct 8-byte bank slots: rows 2a and 2(a ^ 8) + 1 collide.  Odd
// rows are therefore stored 8 bytes further on (logical byte b of the row at
// byte b + 8), which sets bit 3 of the slot from the row parity and makes
// the read conflict-free.  A shifted row spills 8 bytes into a seventh unit
// at each end; the loads fill both edges from the neighbouring bytes of the
// operand, which exist for every row but the operand's last.  The rows of a
// tile whose index within its 32-row block equals `unshifted` (the block
// position of the operand's last row, or 32 for none) are not shifted.
SG_HD uint32_t mxfp6_lds_offset(uint32_t row, uint32_t byte, uint32_t unshifted) {
  const uint32_t b = byte + (((row & 1u) && (row & 31u) != unshifted) ? 8u : 0u);
  return lds_offset<128, kSwzDefault>(row, b >> 4) + (b & 15u);
}

// An MN-major B half tile of the 256x256 kernel of 16x16x32 MFMAs: one
// 256-byte LDS row per k (128 n values), its 32-byte units (16 n) placed at
// unit XOR mn256_key(k).  A fragment read (ds_read_b64_tr_b16) covers, per
// 32 lanes, rows k0..k0+3 and k0+8..k0+11 at one 32-byte unit; the key
// gives those eight rows eight different units, so the read meets the 64
// banks once.  Returns the byte offset of byte `byte` of row k.
SG_HD constexpr uint32_t mn256_key(uint32_t k) { return (k & 3u) | (((k >> 3) & 1u) << 2); }
SG_HD constexpr uint32_t mn256_lds_offset(uint32_t k, uint32_t byte) {
  return k * 256u + 32u * ((byte >> 5) ^ mn256_key(k)) + (byte & 31u);
}

// The C block that the 256x256 kernel of 16x16x32 MFMAs brings into LDS
// through the loads of its last two K tiles (a 16-bit C): wave w4 of a
// group owns 128 output rows x 64 columns, and row r, 16-byte chunk c (8
// columns) of that block lies in quarter r / 32, one 16 KiB half slot of the
// operand rings, in the wave's 1 KiB region 4((r / 8) mod 4) + w4, where a
// direct-to-LDS load puts lane l's 16 bytes at byte 16 l: row r mod 8 (128
// bytes), chunk c XOR cblock_key(r).  The key spreads the 16 rows that one
// 8-byte epilogue read covers (rows R..R+15, one chunk half) over the 16
// chunk positions of a 256-byte bank line, so 32 lanes touch 64 banks once.
// Returns quarter * 16384 + the offset inside the quarter's half slot.
// With swz = false the chunk keeps its logical place (the output half of the
// layout ablation).
SG_HD constexpr uint32_t cblock_key(uint32_t r) { return (r >> 1) & 7u; }
SG_HD constexpr uint32_t cblock_lds_offset(uint32_t w4, uint32_t r, uint32_t c,
                                           bool swz = true) {
  return (r >> 5) * 16384u + (4u * ((r >> 3) & 3u) + w4) * 1024u + (r & 7u) * 128u +
         16u * (c ^ (swz ? cblock_key(r) : 0u));
}

}  // namespace sg
