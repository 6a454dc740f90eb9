// pingpong.h -- the 8-wave "ping-pong" mainloop for 256x256 tiles whose A
// and B are both K-major: 16-bit elements with 32x32x16 MFMAs here (the
// 16x16x32 form is pingpong16.h), and the block-scaled MXFP8 / MXFP6 / MXFP4
// form at the end of this file.
//
// Roles.  The workgroup's 8 waves form two groups of four, one wave of each
// group per SIMD (the hardware deals a workgroup's waves to the SIMDs round
// robin, so waves w and w+4 share a SIMD).  Group g owns output rows
// [128g, 128g+128); wave w4 of a group owns columns [64 w4, 64 w4 + 64), the
// same 4x2 grid of 32x32 accumulators as the 8-wave GemmTile.  The groups
// run the same program one phase apart: in every phase one wave of each
// SIMD issues 16 MFMAs back to back from registers (and, between them, its
// share of the global -> LDS loads), while the other reads its next
// fragments from LDS; a workgroup barrier ends every phase and the two swap
// roles.  A phase covers 32 of K, so a 64-wide K tile takes four phases.
//
// LDS (160 KiB).  A K tile of one operand is two halves of 128 rows x 128
// bytes (16 KiB, under the swizzle lds_offset<128, 16>): rows 0..127 and
// 128..255.  A lives in a ring of two tiles, B in a ring of three.  Group g
// loads the g-th half of every tile of both operands, so each load moves
// whole 128-byte row segments (one cache line) -- measured faster than
// 64-byte segments -- and the loads go out evenly, four per compute phase:
//   compute phase over the first K half of tile t:  B half of tile t+2,
//   compute phase over the second K half of tile t: A half of tile t+2.
// A half of tile t is read only by its own group (output rows), so its slot
// is free once that group's second memory phase of tile t is over; B slot
// (t+2) mod 3 held tile t-1.  Every load has five to seven phases to land.
//
// The direct-to-LDS loads are written as inline assembly: the compiler then
// neither tracks them (it would otherwise make every LDS read wait for all
// loads in flight, as it cannot tell the ring slots apart) nor reorders LDS
// reads across them; the waits are explicit.
#pragma once

#include <type_traits>

#include "gemm_kernels.h"
#include "mx_kernels.h"

namespace sg {

// Buffer descriptor as four SGPRs (raw access, stride 0, range-checked).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at byte `voff` of the
// buffer go to LDS address m0 + 16 l.  `lds` must be wave-uniform.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen lds"
      :
      : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(rsrc)
      : "memory", "m0");
}

// buffer_load_dwordx4 ... lds with the LDS address m0 = lds_base + imm and an
// SGPR byte offset `soff` added to the global address (three instructions:
// the m0 write, the wait state it needs, the load).
template <int Imm>
__device__ __forceinline__ void dma16_so(u32x4 rsrc, uint32_t voff, uint32_t soff,
                                         uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %1, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, %3 offen lds"
      :
      : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(rsrc),
        "s"(__builtin_amdgcn_readfirstlane(soff)), "i"(Imm)
      : "memory", "m0", "scc");
}

// The same load split in two: set_m0 writes m0 = lds_base + Imm, and
// dma16_so_m0 issues the load with whatever m0 holds.  A kernel that places
// the m0 write an MFMA ahead of its load (nothing in between may write m0)
// keeps the wave's MFMA stream moving: measured on MI355X, an LDS-DMA load
// right after its m0 write and wait state delays the wave's next MFMA by
// about 14 cycles, one issued an MFMA after the write by about 7.
template <int Imm>
__device__ __forceinline__ void set_m0(uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %0, %1"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "i"(Imm)
               : "m0", "scc");
}
__device__ __forceinline__ void dma16_so_m0(u32x4 rsrc, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

// buffer_load_dword ... lds: lane l's 4 bytes at byte `voff` go to LDS
// address m0 + 4 l.
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %2, 0 offen lds"
      :
      : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(rsrc)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global -> LDS loads of one half tile (128 rows x 128 bytes of K)
// by the four waves of a group: 16 regions of 1 KiB, wave w4 fills regions
// 4i + w4.  Lane l of a region fills physical bytes [16l, 16l+16) of it,
// the logical chunk whose swizzled offset that is; regions 4 KiB apart share
// the XOR key, so the lane's row advances by 32 per region and its 16-byte
// K chunk stays fixed.
template <int Swz>
struct HalfLoader {
  uint32_t base;   // row * pitch + chunk byte
  uint32_t chunk;  // byte of K inside the tile (0, 16, ..., 112)
  uint32_t pitch;
  int row;         // row of region w4 inside the half

  __device__ __forceinline__ void init(int w4, int lane, uint32_t row_pitch) {
    const uint32_t phys = (uint32_t)w4 * 1024u + 16u * (uint32_t)lane;
    const uint32_t logical = swz_bytes<Swz>(phys);
    row = (int)(logical >> 7);
    chunk = logical & 127u;
    pitch = row_pitch;
    base = (uint32_t)row * row_pitch + chunk;
  }

  // Load i (0..3) of K bytes [kbyte0, kbyte0 + 128) into the half at LDS
  // address `half` (+ the region); rows at or beyond rows_valid and bytes at
  // or beyond kbytes_total read as zero.
  __device__ __forceinline__ void issue(u32x4 rsrc, uint32_t half, int w4, int i,
                                        int rows_valid, uint32_t kbyte0,
                                        uint32_t kbytes_total) const {
    const bool ok = kbyte0 + chunk < kbytes_total && row + 32 * i < rows_valid;
    const uint32_t off = ok ? base + (uint32_t)(32 * i) * pitch + kbyte0 : kOutOfRange;
    dma16(rsrc, off, half + (uint32_t)(4 * i + w4) * 1024u);
  }
  // issue in two steps (set_m0): the m0 write, then the load.
  __device__ __forceinline__ void prep(uint32_t half, int w4, int i) const {
    set_m0<0>(half + (uint32_t)(4 * i + w4) * 1024u);
  }
  __device__ __forceinline__ void go(u32x4 rsrc, int i, int rows_valid, uint32_t kbyte0,
                                     uint32_t kbytes_total) const {
    const bool ok = kbyte0 + chunk < kbytes_total && row + 32 * i < rows_valid;
    const uint32_t off = ok ? base + (uint32_t)(32 * i) * pitch + kbyte0 : kOutOfRange;
    dma16_so_m0(rsrc, off, 0u);
  }
};

// The half-tile loader for K a multiple of 64: each lane's four row offsets
// (out of range for rows past the operand) are fixed per tile job, and the K
// position of a load travels in the instruction's SGPR offset; a K tile past
// the end is loaded through a descriptor with no records (zero fill).
template <int Swz>
struct KExactHalfLoader {
  uint32_t voff[4];

  __device__ __forceinline__ void init(const HalfLoader<Swz>& h, int rows_valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      voff[i] = h.row + 32 * i < rows_valid ? h.base + (uint32_t)(32 * i) * h.pitch
                                            : kOutOfRange;
  }

  template <int I>
  __device__ __forceinline__ void issue(u32x4 rsrc, uint32_t half, int w4,
                                        uint32_t kbyte0) const {
    dma16_so<I * 4096>(rsrc, voff[I], kbyte0, half + (uint32_t)w4 * 1024u);
  }
  // issue<I> in two steps, m0 first (see set_m0).
  template <int I>
  __device__ __forceinline__ void prep(uint32_t half, int w4) const {
    set_m0<I * 4096>(half + (uint32_t)w4 * 1024u);
  }
  template <int I>
  __device__ __forceinline__ void go(u32x4 rsrc, uint32_t kbyte0) const {
    dma16_so_m0(rsrc, voff[I], kbyte0);
  }
};

// The four 16 KiB half slots of group g that hold a wave's block of C or D
// at the end of a 256x256 tile (cblock_lds_offset's quarters): the slots
// the loads of K tiles T and T+1 fill, B ring (after A's two slots) and A
// ring alternating.
__device__ __forceinline__ void cblock_quarters(char* (&cq)[4], char* smem, int T, int g,
                                                int tile_bytes, int half_bytes) {
  const int tb = T % 3, ta = T & 1;
  char* const b_slots = smem + 2 * tile_bytes + g * half_bytes;
  char* const a_slots = smem + g * half_bytes;
  cq[0] = b_slots + tb * tile_bytes;
  cq[1] = a_slots + ta * tile_bytes;
  cq[2] = b_slots + (tb == 2 ? 0 : tb + 1) * tile_bytes;
  cq[3] = a_slots + (ta ^ 1) * tile_bytes;
}

// Where the 256x256 kernel of 16x16x32 MFMAs stages a 16-bit D: wave w4's
// own 1 KiB regions of the four quarters (as the C block: row r of its 128 x
// 64 block in quarter r / 32, region 4((r / 8) mod 4) + w4, 128-byte row r
// mod 8), 16-byte chunk c at chunk c XOR (r mod 8), so that the 8 rows of a
// ds_write_b128 phase fill one 128-byte bank line.  Offset inside the
// quarter's 16 KiB half slot.  With Swz false the chunk keeps its logical
// place (the output half of the layout ablation).
template <bool Swz = true>
__device__ __forceinline__ uint32_t dstage_offset(uint32_t w4, uint32_t r, uint32_t c) {
  return (4u * ((r >> 3) & 3u) + w4) * 1024u + (r & 7u) * 128u +
         16u * (c ^ (Swz ? (r & 7u) : 0u));
}

// Stores wave w4's staged 128 x 64 block of a 16-bit D: lane l takes 16-byte
// chunk l%8 of row 8s + l/8 (one contiguous KiB per read), so 8 lanes store
// one 128-byte row segment (16 stores per wave).  N is a multiple of 4: a
// chunk with 4 valid columns stores its first 8 bytes.
template <bool OutSwz = true>
__device__ __forceinline__ void store_d16_block(char* const (&cq)[4], const TileJob& j, void* D,
                                                int64_t ldd, int lane, int g, int w4) {
  const int cc = lane & 7;
  const int nl = 64 * w4 + 8 * cc;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const uint32_t r = (uint32_t)(8 * s + (lane >> 3));
    const u32x4 d = lds_read16(cq[s >> 2], dstage_offset<OutSwz>((uint32_t)w4, r, (uint32_t)cc));
    const int ml = 128 * g + (int)r;
    if (ml >= j.m_valid || nl >= j.n_valid) continue;
    uint16_t* p = static_cast<uint16_t*>(D) + (j.d_row0 + ml) * ldd + j.n0 + nl;
    if (j.n_valid - nl >= 8)
      *reinterpret_cast<u32x4*>(p) = d;
    else
      *reinterpret_cast<u32x2*>(p) = u32x2{d[0], d[1]};
  }
}

template <bool IsBF16, int Swz>
struct PingPongTile {
  using Base = GemmTile<256, 256, IsBF16, false, false, Swz, 8>;
  static constexpr int kHalfBytes = 16384;             // 128 rows x 128 B
  static constexpr int kTileBytes = 2 * kHalfBytes;    // one operand, one K tile
  static constexpr int kBK = 64;
  static constexpr int kARing = 2, kBRing = 3;
  static constexpr int kLdsBytes = (kARing + kBRing) * kTileBytes;  // 160 KiB
  static constexpr int kFM = 4, kFN = 2;               // 32x32 blocks per wave
  static_assert(Base::kFM == kFM && Base::kFN == kFN, "wave grid must match the epilogue");

  // Fragments of one 32-wide K half (two 16-wide K steps).
  struct Frags {
    u32x4 a[2][kFM], b[2][kFN];
  };

  // Per-lane byte offsets, inside an operand's K tile, of fragment 0 for
  // each K half and 16-wide step; fragment f is f * 4096 bytes further (32
  // LDS rows, the same XOR key).
  struct Offsets {
    uint32_t a[2][2], b[2][2];
  };

  __device__ __forceinline__ static Offsets offsets(int g, int w4, int lrow, int lhalf) {
    Offsets o;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint32_t c = 4 * kh + 2 * kk + lhalf;
        o.a[kh][kk] = g * kHalfBytes + lds_offset<128, Swz>(lrow, c);
        o.b[kh][kk] = (w4 >> 1) * kHalfBytes + lds_offset<128, Swz>((w4 & 1) * 64 + lrow, c);
      }
    return o;
  }

  __device__ __forceinline__ static void read(Frags& f, const char* at, const char* bt,
                                              const Offsets& o, int kh) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int fm = 0; fm < kFM; ++fm) f.a[kk][fm] = lds_read16(at, o.a[kh][kk] + fm * 4096);
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) f.b[kk][fn] = lds_read16(bt, o.b[kh][kk] + fn * 4096);
    }
  }

  // 16 MFMAs with the four loads of one half tile between them, one per
  // four MFMAs (without the MFMAs for a wave whose output rows are all past
  // M: it still loads its share of B and keeps the barriers).
  template <bool Active>
  __device__ __forceinline__ static void compute(f32x16 (&acc)[kFM][kFN], const Frags& f,
                                                 const HalfLoader<Swz>& ld, u32x4 rsrc,
                                                 uint32_t half, int w4, int rows_valid,
                                                 uint32_t kbyte0, uint32_t kbytes) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = q >> 1;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int fm = ((q & 1) << 1) | (m >> 1), fn = m & 1;
        if constexpr (Active)
          acc[fm][fn] = mfma32x32x16<IsBF16>(f.b[kk][fn], f.a[kk][fm], acc[fm][fn]);
      }
      __builtin_amdgcn_sched_barrier(0);
      ld.issue(rsrc, half, w4, q, rows_valid, kbyte0, kbytes);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Workgroup barrier that waits for nothing: loads stay in flight across
  // it (the waits are explicit) and the compiler moves no memory access
  // across it.
  __device__ __forceinline__ static void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // The end of every phase: the wave's LDS reads have returned (no later
  // load may overwrite a slot under them) and all but its 8 newest loads
  // (two half tiles) have landed.  The 8 newest are the halves of the two
  // K tiles after the next one to be read, so before each barrier the wave
  // has its share of every tile a later phase reads next in LDS.
  __device__ __forceinline__ static void end_phase() {
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    barrier();
  }

  template <bool Active>
  __device__ __forceinline__ static void mainloop(f32x16 (&acc)[kFM][kFN],
                                                  const HalfLoader<Swz>& la,
                                                  const HalfLoader<Swz>& lb, u32x4 ra, u32x4 rb,
                                                  int a_rows, int b_rows, uint32_t a_ring,
                                                  uint32_t b_ring, const char* a_rd,
                                                  const char* b_rd, const Offsets& o, int g,
                                                  int w4, int T, uint32_t kbytes) {
    if (g) barrier();  // group 1 runs one phase behind group 0
    int bs = 0;        // t mod 3
    for (int t = 0; t < T; ++t) {
      const int as = t & 1, bs2 = bs == 0 ? 2 : bs - 1;  // (t+2) mod 2, (t+2) mod 3
      const char* at = a_rd + as * kTileBytes;
      const char* bt = b_rd + bs * kTileBytes;
      const uint32_t k2 = (uint32_t)(t + 2) * 128u;
      Frags f;
      if constexpr (Active) read(f, at, bt, o, 0);
      end_phase();
      compute<Active>(acc, f, lb, rb, b_ring + bs2 * kTileBytes, w4, b_rows, k2, kbytes);
      end_phase();
      if constexpr (Active) read(f, at, bt, o, 1);
      end_phase();
      compute<Active>(acc, f, la, ra, a_ring + as * kTileBytes, w4, a_rows, k2, kbytes);
      end_phase();
      bs = bs == 2 ? 0 : bs + 1;
    }
    if (!g) barrier();
  }

  // Mainloop and epilogue of one tile; `smem` is the 160 KiB of LDS.
  __device__ __forceinline__ static void run(char* smem, const TileJob& j, int64_t K,
                                             const void* C, int c_dtype, void* D,
                                             int d_dtype, int64_t ldd) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, w4 = wave & 3;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // Group g loads rows [128g, 128g+128) of both operands.
    const u32x4 ra = rsrc_words(j.a, j.a_bytes), rb = rsrc_words(j.b, j.b_bytes);
    const int a_rows = j.m_valid - 128 * g, b_rows = j.n_valid - 128 * g;
    HalfLoader<Swz> la, lb;
    la.init(w4, lane, j.a_pitch);
    lb.init(w4, lane, j.b_pitch);
    la.base += (uint32_t)(128 * g) * j.a_pitch;
    lb.base += (uint32_t)(128 * g) * j.b_pitch;

    const uint32_t s0 = lds_addr(smem);
    const uint32_t a_ring = s0 + g * kHalfBytes;                       // + (t%2) tiles
    const uint32_t b_ring = s0 + kARing * kTileBytes + g * kHalfBytes; // + (t%3) tiles
    const char* a_rd = smem;
    const char* b_rd = smem + kARing * kTileBytes;

    const uint32_t kbytes = (uint32_t)K * 2u;
    const int T = (int)((K + kBK - 1) / kBK);

    // Tiles 0 and 1 (B before A, the order the mainloop keeps).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lb.issue(rb, b_ring + t * kTileBytes, w4, i, b_rows, t * 128u, kbytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        la.issue(ra, a_ring + t * kTileBytes, w4, i, a_rows, t * 128u, kbytes);
    }
    end_phase();

    const Offsets o = offsets(g, w4, lrow, lhalf);
    f32x16 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int k = 0; k < kFN; ++k) acc[i][k] = f32x16{};

    // A wave whose 128 output rows all lie past M (the second group of a tile
    // with at most 128 valid rows) runs the mainloop without its MFMAs.
    if (a_rows > 0)
      mainloop<true>(acc, la, lb, ra, rb, a_rows, b_rows, a_ring, b_ring, a_rd, b_rd, o, g, w4,
                     T, kbytes);
    else
      mainloop<false>(acc, la, lb, ra, rb, a_rows, b_rows, a_ring, b_ring, a_rd, b_rd, o, g,
                      w4, T, kbytes);
    wait_vmem();  // the zero-filled loads past K

    Base::epilogue(acc, j, C, c_dtype, D, d_dtype, ldd, lane, g, w4);
  }
};

template <bool IsBF16, int Swz>
__global__ void __launch_bounds__(512, 1) pingpong_gemm_kernel(const DenseParams p) {
  using Tile = PingPongTile<IsBF16, Swz>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = dense_tile_job<256, 256, false, false>(p, blockIdx.x);
  Tile::run(smem, j, p.K, p.C, p.c_dtype, p.D, p.d_dtype, p.ldd);
  clock_end(p.clk, cs);
}

}  // namespace sg

namespace sg {

// The ping-pong mainloop for the block-scaled GEMMs: MXFP8 (e4m3 elements),
// MXFP6 (e2m3 or e3m2 elements, a 6-bit stream) and MXFP4 (e2m1 elements,
// two per byte).  A K tile is 128 bytes of every row for MXFP8 and MXFP4
// (128 e4m3 or 256 e2m1 values: four or eight 32-element scale blocks), so
// the operand halves have exactly the geometry of the 16-bit kernel's; for
// MXFP6 it is 96 bytes (128 values), kept in the same 128-byte LDS rows
// under mxfp6_lds_offset.
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (checked on the GPU
// with one-hot operands): lane l supplies row l%32; with e4m3 its 32 bytes
// are K [16h, 16h+16) and [32+16h, 32+16h+16) of the 64-wide step, with e2m1
// its first 16 bytes are the 32 values of block h of the step, with e2m3 or
// e3m2 its first 24 bytes are the 32 values of block h as a 6-bit stream
// (h = l/32; the remaining bytes are ignored); the e8m0 byte of lane l
// scales block h.  So a lane reads 16-byte chunk 4kk + 2c + h of the row for
// chunk c of e4m3 step kk, or for step 2kk + c of e2m1: one offset table
// serves both; for e2m3/e3m2 step kk it reads bytes [24(2kk + h), +24).  A
// phase is eight e4m3 or fp6 MFMAs (one 64-wide step) or sixteen e2m1 MFMAs
// (two steps): 512 cycles of MFMA for e4m3 and e2m1, 256 for fp6 (the
// 6-bit MFMA runs at the 4-bit rate).
//
// Schedule: the 16-bit ping-pong's for K a multiple of 64 (pingpong16.h).
// LDS holds an A ring of two tiles and a B ring of three (160 KiB); group g
// loads half g of every tile of both operands, from its memory phases after
// their reads: A(t+1) in the one over the first K step of tile t, B(t+2) in
// the one over the second, so the compute phases are MFMAs only (and the
// scale loads below); both groups run the same instruction stream.  The
// e8m0 scales do not fit in LDS beside the rings: each wave loads the
// scale dwords of its own rows (four A rows and two B rows per lane, one or
// two dwords each) straight into registers, with the A half of the first
// tile of a group, for the next group.
//
// Fmt is the MFMA's operand format code: 0 e4m3, 2 e2m3, 3 e3m2, 4 e2m1.
// Blocks: the scales come in the 64-row block layout (SG_SF_BLOCKS), whose
// 16 bytes for a row and a group of 16 blocks hold the 8 even blocks, then
// the 8 odd ones.  Lane half h of the MFMA scales block 2s + h of step s, so
// one lane-half swap per group (take) leaves each lane the 8 bytes it needs
// and the MFMA gets the dword as it stands, the op-select naming the byte;
// in the rows layout every phase swaps and shifts (pick_scales).
template <int Swz, int Fmt, bool Blocks>
struct PingPongMxTile {
  static_assert(Fmt == 0 || Fmt == 2 || Fmt == 3 || Fmt == 4, "operand format");
  static constexpr bool kFp4 = Fmt == 4, kFp6 = Fmt == 2 || Fmt == 3;
  static_assert(!kFp6 || Swz == kSwzDefault, "the fp6 layout is built on the default swizzle");
  using Base = GemmTile<256, 256, true, false, false, Swz, 8>;
  static constexpr int kHalfBytes = 16384;
  static constexpr int kTileBytes = 2 * kHalfBytes;
  static constexpr int kBK = kFp4 ? 256 : 128;             // elements of K per tile
  static constexpr int kTileRowBytes = kFp6 ? 96 : 128;    // bytes of a row per tile
  static constexpr int kScaleDw = kFp4 ? 2 : 1;            // scale dwords per row per tile
  static constexpr int kARing = 2, kBRing = 3;
  static constexpr int kLdsBytes = (kARing + kBRing) * kTileBytes;  // 160 KiB
  static constexpr int kMfmas = kFp4 ? 16 : 8;             // per compute phase
  static constexpr int kFM = 4, kFN = 2;
  static constexpr int kPieces = kFp6 ? 3 : 2;             // LDS reads per fragment
  // Scales: a 16-byte load covers kScaleTiles K tiles (four for e4m3 and
  // fp6, two for e2m1 with its two dwords a tile) of 64 scale rows: lanes
  // 0-31 take the rows of one 32-row fragment block, lanes 32-63 those of
  // the next (A blocks 0|1 and 2|3, B blocks 0|1), and a swap of the lane
  // halves gives every lane both (once per group in the block layout, where
  // each lane keeps only its own half of the 16 bytes; per phase in the rows
  // layout).
  static constexpr int kScaleTiles = kFp4 ? 2 : 4;
  static constexpr int kScaleLoads = 3;  // per wave and scale group

  // One phase's fragments: e4m3/e2m1 chunk c of every 32-row block (16
  // bytes), or fp6 piece q (8 bytes) of the lane's 24.
  using Piece = typename std::conditional<kFp6, u32x2, u32x4>::type;
  struct Frags {
    Piece a[kFM][kPieces], b[kFN][kPieces];
  };

  struct Offsets {
    uint32_t a[2][kPieces], b[2][kPieces];  // [kk][c or q]
  };

  // The raw scale dwords of one scale group as loaded: [block pair], dword
  // kScaleDw * (tile within the group) + d in the rows layout; in the block
  // layout dwords 0-1 hold the even blocks, 2-3 the odd ones.
  struct Scales {
    u32x4 a[2], b;
  };
  // The block layout's group once its lane halves are swapped: [fragment
  // block], dword (tile within the group) / 2 for e4m3 and fp6, tile within
  // the group for e2m1, of the lane's half (even blocks in lanes 0-31, odd
  // ones in lanes 32-63).
  struct BlockScales {
    u32x2 a[kFM], b[kFN];
  };
  // The group the compute phases use.
  using Cur = typename std::conditional<Blocks, BlockScales, Scales>::type;

  // `ua`, `ub`: the block position of the rows that mxfp6_lds_offset leaves
  // unshifted (fp6 only).
  __device__ __forceinline__ static Offsets offsets(int g, int w4, int lrow, int lhalf,
                                                    uint32_t ua, uint32_t ub) {
    Offsets o;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int c = 0; c < kPieces; ++c) {
        if constexpr (kFp6) {
          const uint32_t byte = 24u * (2 * kk + lhalf) + 8u * c;
          o.a[kk][c] = g * kHalfBytes + mxfp6_lds_offset(lrow, byte, ua);
          o.b[kk][c] = (w4 >> 1) * kHalfBytes + mxfp6_lds_offset((w4 & 1) * 64 + lrow, byte, ub);
        } else {
          const uint32_t ch = 4 * kk + 2 * c + lhalf;
          o.a[kk][c] = g * kHalfBytes + lds_offset<128, Swz>(lrow, ch);
          o.b[kk][c] = (w4 >> 1) * kHalfBytes + lds_offset<128, Swz>((w4 & 1) * 64 + lrow, ch);
        }
      }
    return o;
  }

  __device__ __forceinline__ static Piece read_piece(const char* t, uint32_t off) {
    if constexpr (kFp6)
      return lds_read8(t, off);
    else
      return lds_read16(t, off);
  }

  __device__ __forceinline__ static void read(Frags& f, const char* at, const char* bt,
                                              const Offsets& o, int kk) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int c = 0; c < kPieces; ++c) f.a[fm][c] = read_piece(at, o.a[kk][c] + fm * 4096);
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
      for (int c = 0; c < kPieces; ++c) f.b[fn][c] = read_piece(bt, o.b[kk][c] + fn * 4096);
  }

  // Scale load q (0 .. 2) of the group at byte offset `soff` (from a row's
  // first scale byte): A block pair q, or the B block pair.  Rows layout:
  // the offset goes into the range-checked VGPR offset, as a group's last 16
  // bytes may run past the end of the operand's last row.  Block layout: a
  // group's 16 bytes lie inside the array for every row the descriptor
  // covers, so the offset travels in an SGPR.  Compiler-tracked buffer
  // loads: the first use of the registers waits for them.
  __device__ __forceinline__ static void load_scale(Scales& s, int q,
                                                    __amdgpu_buffer_rsrc_t rsa,
                                                    __amdgpu_buffer_rsrc_t rsb,
                                                    const uint32_t (&va)[2], uint32_t vb,
                                                    uint32_t soff) {
    if constexpr (Blocks) {
      if (q < 2)
        s.a[q] = buffer_load16_so(rsa, va[q], soff);
      else
        s.b = buffer_load16_so(rsb, vb, soff);
    } else {
      if (q < 2)
        s.a[q] = buffer_load16(rsa, va[q] + soff);
      else
        s.b = buffer_load16(rsb, vb + soff);
    }
  }

  // cur = nxt as an ordered step: each register set passes through an
  // empty statement tied to its own registers, which no LDS read or load
  // may cross, so the copy (and any wait the compiler puts before its
  // first use of `nxt`) comes where it is written.  Block layout: lane l
  // holds a row of block 2p (l < 32) or 2p + 1 (l >= 32), even blocks in
  // dwords 0-1 and odd ones in 2-3; swapping the odd dwords of lanes 0-31
  // with the even dwords of lanes 32-63 leaves in every lane the half that
  // lane half scales, of block 2p in one register and of 2p + 1 in the other.
  __device__ __forceinline__ static void take(Cur& cur, Scales& nxt) {
    asm volatile("" : "+v"(nxt.a[0]) : : "memory");
    asm volatile("" : "+v"(nxt.a[1]) : : "memory");
    asm volatile("" : "+v"(nxt.b) : : "memory");
    if constexpr (Blocks) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const auto r = __builtin_amdgcn_permlane32_swap(nxt.a[p][k], nxt.a[p][k + 2], false,
                                                          false);
          cur.a[2 * p][k] = r[0];
          cur.a[2 * p + 1][k] = r[1];
        }
        const auto r = __builtin_amdgcn_permlane32_swap(nxt.b[k], nxt.b[k + 2], false, false);
        cur.b[0][k] = r[0];
        cur.b[1][k] = r[1];
      }
    } else {
      cur = nxt;
    }
    settle(cur);
  }

  // A use of the scale registers at this point of the program.
  __device__ __forceinline__ static void settle(Scales& s) {
    asm volatile("" : "+v"(s.a[0]) : : "memory");
    asm volatile("" : "+v"(s.a[1]) : : "memory");
    asm volatile("" : "+v"(s.b) : : "memory");
  }
  __device__ __forceinline__ static void settle(BlockScales& s) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) asm volatile("" : "+v"(s.a[i]) : : "memory");
#pragma unroll
    for (int i = 0; i < kFN; ++i) asm volatile("" : "+v"(s.b[i]) : : "memory");
  }

  // The scale registers of compute phase `ph` (0, 1) of tile `sub` of the
  // group.  Rows layout: dword w = kScaleDw sub (+ ph for e2m1) of the
  // wave's rows; a lane-half swap turns a pair's register (block 2p in
  // lanes 0-31, 2p+1 in lanes 32-63) into one per block holding it in all
  // lanes; then the lane's block (lane half) is shifted into the even bytes
  // so that op-select 2c picks block 2c + h.  Block layout: the loaded
  // dword (see sel0).
  __device__ __forceinline__ static void pick_scales(uint32_t (&sa)[kFM], uint32_t (&sb)[kFN],
                                                     const Cur& s, int sub, int ph,
                                                     int lhalf) {
    if constexpr (Blocks) {
      const int w = kFp4 ? sub : sub >> 1;
#pragma unroll
      for (int fm = 0; fm < kFM; ++fm) sa[fm] = s.a[fm][w];
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) sb[fn] = s.b[fn][w];
    } else {
      const int w = kScaleDw * sub + (kFp4 ? ph : 0);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const auto r = __builtin_amdgcn_permlane32_swap(s.a[p][w], s.a[p][w], false, false);
        sa[2 * p] = r[0] >> (8 * lhalf);
        sa[2 * p + 1] = r[1] >> (8 * lhalf);
      }
      const auto r = __builtin_amdgcn_permlane32_swap(s.b[w], s.b[w], false, false);
      sb[0] = r[0] >> (8 * lhalf);
      sb[1] = r[1] >> (8 * lhalf);
    }
  }

  // One scaled MFMA on 8-dword operands.
  template <int Sel>
  __device__ __forceinline__ static f32x16 mfma(const i32x8& av, const i32x8& bv, f32x16 acc,
                                                uint32_t sa, uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc, Fmt, Fmt, Sel, (int)sb,
                                                           Sel, (int)sa);
  }

  // The operand of one MFMA: e4m3 both chunks of the step; e2m1 chunk c
  // (the upper 16 bytes are ignored); fp6 the three pieces (the last 8
  // bytes are ignored).
  __device__ __forceinline__ static i32x8 operand(const Piece (&p)[kPieces], int c) {
    if constexpr (kFp6) {
      const u32x4 lo = __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3);
      const u32x4 hi = __builtin_shufflevector(p[2], p[2], 0, 1, -1, -1);
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if constexpr (kFp4) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(p[c], z, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  // The op-select (scale byte) of the MFMAs of compute phase `ph` of tile
  // `sub` of the group: rows layout, byte 2 ph (e4m3, fp6: the phase's
  // step) or byte 2c (e2m1: chunk c, added in compute) of the shifted
  // dword; block layout, where block 2s + h of the phase's step s sits in
  // the lane's half: byte 2 (sub mod 2) + ph (e4m3, fp6) or 2 ph + c (e2m1).
  __device__ __forceinline__ static constexpr int sel0(int sub, int ph) {
    return Blocks ? (kFp4 ? 2 * ph : 2 * (sub & 1) + ph) : (kFp4 ? 0 : 2 * ph);
  }
  static constexpr int kSelPerChunk = Blocks ? 1 : 2;  // e2m1

  // kMfmas MFMAs of one compute phase, op-select sel0 (+ the chunk's share
  // for e2m1); N loads go out spread between them, the first after the
  // first MFMA, at most one after each MFMA.  `prep(q)` (the m0 write of a
  // direct-to-LDS load, see set_m0) runs before the MFMA that load q
  // follows, `go(q)` issues the load after it.
  template <int N, class Prep, class Go>
  __device__ __forceinline__ static void compute(f32x16 (&acc)[kFM][kFN], const Frags& f,
                                                 const uint32_t (&sa)[kFM],
                                                 const uint32_t (&sb)[kFN], int sel0,
                                                 const Prep& prep, const Go& go) {
    static_assert(N <= kMfmas, "one load per MFMA");
#pragma unroll
    for (int m = 0; m < kMfmas; ++m) {
      const int c = m / (kFM * kFN), fm = (m >> 1) % kFM, fn = m & 1;
      const i32x8 av = operand(f.a[fm], c), bv = operand(f.b[fn], c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < N; ++q)
        if (q * kMfmas / N == m) prep(q);
      __builtin_amdgcn_sched_barrier(0);
      const int sel = sel0 + (kFp4 ? kSelPerChunk * c : 0);
      if (sel == 0)
        acc[fm][fn] = mfma<0>(av, bv, acc[fm][fn], sa[fm], sb[fn]);
      else if (sel == 1)
        acc[fm][fn] = mfma<1>(av, bv, acc[fm][fn], sa[fm], sb[fn]);
      else if (sel == 2)
        acc[fm][fn] = mfma<2>(av, bv, acc[fm][fn], sa[fm], sb[fn]);
      else
        acc[fm][fn] = mfma<3>(av, bv, acc[fm][fn], sa[fm], sb[fn]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < N; ++q)
        if (q * kMfmas / N == m) go(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ static void barrier() { PingPongTile<true, Swz>::barrier(); }

  // The end of a phase of the mainloop: the wave's LDS reads have returned
  // (Lgkm) and all but its V newest loads have landed (V < 0: no load wait),
  // then the barrier.
  template <int V, bool Lgkm>
  __device__ __forceinline__ static void sync() {
    static_assert(V >= -1 && V < 64, "vmcnt immediate");
    if constexpr (V >= 0 && Lgkm)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(V) : "memory");
    else if constexpr (V >= 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V) : "memory");
    else if constexpr (Lgkm)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
  }

  // The fp6 half-tile loader.  The physical slots a lane fills are those of
  // HalfLoader; slot j of logical row r receives the operand bytes
  // [16j - 8s, 16j - 8s + 16) of the K tile, s = 1 for a shifted row
  // (mxfp6_lds_offset).  Slots holding none of the tile's 96 bytes are not
  // loaded (out of range: zero fill, no traffic); so are rows past the
  // operand.  The row offsets are fixed per tile job; the K position travels
  // in the SGPR offset; tiles past the end load through an empty descriptor.
  struct Fp6Loader {
    uint32_t voff[4];

    __device__ __forceinline__ void init(int w4, int lane, uint32_t pitch, int rows_valid,
                                         uint32_t unshifted) {
      HalfLoader<Swz> h;
      h.init(w4, lane, pitch);
      const uint32_t s = ((h.row & 1) && (uint32_t)h.row != unshifted) ? 8u : 0u;
      const uint32_t j = h.chunk >> 4;
      const bool used = 16u * j < 96u + s;  // the slot holds some of bytes [0, 96)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        voff[i] = used && h.row + 32 * i < rows_valid
                      ? (uint32_t)(h.row + 32 * i) * pitch + 16u * j - s
                      : kOutOfRange;
    }

    template <int I>
    __device__ __forceinline__ void issue(u32x4 rsrc, uint32_t half, int w4,
                                          uint32_t kbyte0) const {
      dma16_so<I * 4096>(rsrc, voff[I], kbyte0, half + (uint32_t)w4 * 1024u);
    }
  };
  using Loader = typename std::conditional<kFp6, Fp6Loader, KExactHalfLoader<Swz>>::type;

  template <class L>
  __device__ __forceinline__ static void issue_half(const L& ld, int i, u32x4 rsrc,
                                                    uint32_t half, int w4, uint32_t kbyte0) {
    if (i == 0) ld.template issue<0>(rsrc, half, w4, kbyte0);
    if (i == 1) ld.template issue<1>(rsrc, half, w4, kbyte0);
    if (i == 2) ld.template issue<2>(rsrc, half, w4, kbyte0);
    if (i == 3) ld.template issue<3>(rsrc, half, w4, kbyte0);
  }

  // ua, ub: fp6 only, see mxfp6_lds_offset.  sfa, sfb: the scales of the
  // tile's first rows, laid out as `sf` says.
  __device__ __forceinline__ static void run(char* smem, const TileJob& j, const char* sfa,
                                             const char* sfb, const SfMap& sf, int64_t K,
                                             void* D, int d_dtype, int64_t ldd, uint32_t ua,
                                             uint32_t ub) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, w4 = wave & 3;
    const int lrow = lane & 31, lhalf = lane >> 5;

    const u32x4 ra = rsrc_words(j.a, j.a_bytes), rb = rsrc_words(j.b, j.b_bytes);
    const u32x4 ra0 = rsrc_words(j.a, 0), rb0 = rsrc_words(j.b, 0);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sfa, sf.tile_bytes(j.m_valid));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sfb, sf.tile_bytes(j.n_valid));
    const int a_rows = j.m_valid - 128 * g, b_rows = j.n_valid - 128 * g;
    Loader la, lb;
    if constexpr (kFp6) {
      la.init(w4, lane, j.a_pitch, a_rows, ua);
      lb.init(w4, lane, j.b_pitch, b_rows, ub);
    } else {
      HalfLoader<Swz> ha, hb;
      ha.init(w4, lane, j.a_pitch);
      hb.init(w4, lane, j.b_pitch);
      la.init(ha, a_rows);
      lb.init(hb, b_rows);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (la.voff[i] != kOutOfRange) la.voff[i] += (uint32_t)(128 * g) * j.a_pitch;
      if (lb.voff[i] != kOutOfRange) lb.voff[i] += (uint32_t)(128 * g) * j.b_pitch;
    }
    // Scale rows of the lane: A 128g + 32(2p + h) + lrow for pair p, B
    // 64 w4 + 32 h + lrow (64 consecutive rows per load: one KiB in the
    // block layout).
    uint32_t sva[2], svb;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 128 * g + 32 * (2 * p + lhalf) + lrow;
      sva[p] = r < j.m_valid ? sf.row((uint32_t)r) : kOutOfRange;
    }
    {
      const int r = 64 * w4 + 32 * lhalf + lrow;
      svb = r < j.n_valid ? sf.row((uint32_t)r) : kOutOfRange;
    }

    const uint32_t s0 = lds_addr(smem);
    const uint32_t a_ring = s0 + g * kHalfBytes;                        // + (t%2) tiles
    const uint32_t b_ring = s0 + kARing * kTileBytes + g * kHalfBytes;  // + (t%3) tiles
    const char* a_rd = smem;
    const char* b_rd = smem + kARing * kTileBytes;
    const int T = (int)(K / kBK);

    auto ld_a = [&](int t, int i) {
      issue_half(la, i, t < T ? ra : ra0, a_ring + (t & 1) * kTileBytes, w4,
                 (uint32_t)t * (uint32_t)kTileRowBytes);
    };
    auto ld_b = [&](int t, int i) {
      issue_half(lb, i, t < T ? rb : rb0, b_ring + (t % 3) * kTileBytes, w4,
                 (uint32_t)t * (uint32_t)kTileRowBytes);
    };
    // Scales of the group starting at tile t (its 16 bytes start at block
    // 4 kScaleDw t, a multiple of 16).  The group after the last (t >= T,
    // loaded but never used) re-reads the last one, so that no offset
    // leaves the array.
    const int t_last = T > 0 ? (T - 1) / kScaleTiles * kScaleTiles : 0;
    auto ld_s = [&](Scales& s, int t, int q) {
      load_scale(s, q, rsa, rsb, sva, svb,
                 sf.block((uint32_t)(min(t, t_last) * 4 * kScaleDw)));
    };

    // Tiles 0 and 1 (B, A, and the scales of the first group: the order the
    // mainloop keeps).  In the rows layout, scale bytes of a group's blocks
    // past K/32 come from the next row or, past the operand, read as zero;
    // no MFMA uses them.  `nxt` receives a group's
    // scales; the group's first memory phase takes them over into `cur`.
    Cur cur;
    Scales nxt;
#pragma unroll
    for (int i = 0; i < 4; ++i) ld_b(0, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) ld_a(0, i);
#pragma unroll
    for (int q = 0; q < kScaleLoads; ++q) ld_s(nxt, 0, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) ld_b(1, i);
    // Tile 0 has landed (B of tile 1 and the scales may be in flight); A of
    // tile 1 comes with the first memory phase.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(4 + kScaleLoads) : "memory");
    barrier();

    const Offsets o = offsets(g, w4, lrow, lhalf, ua, ub);
    f32x16 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int k = 0; k < kFN; ++k) acc[i][k] = f32x16{};

    // Tile t, the Sub-th of its scale group.  The first tile of a group
    // takes the group's scales over from `nxt` and, in its second compute
    // phase, loads the next group's into `nxt`.  The memory phases issue the
    // tile loads after their reads, so the compute phases are MFMAs (and
    // those scale loads) only: A(t+1) into A slot (t+1) mod 2 (its four
    // waves were done with tile t-1 there at the barrier that opened tile t)
    // and B(t+2) into B slot (t+2) mod 3 (both groups were done with tile
    // t-1 there).  Waits, in loads issued after the one waited for: the
    // second memory phase, the other group's B(t+1) for this group's next
    // read (A(t+1), B(t+2) and the scale loads of tile t-1 if it was a
    // group's first); the second compute phase, the wave's own A(t+1)
    // (B(t+2) and this tile's scale loads).
    auto tile = [&](auto sub, int t) {
      constexpr int Sub = decltype(sub)::value;
      constexpr int kWaitM = Sub == 1 ? 8 + kScaleLoads : 8;
      constexpr int kWaitC = Sub == 0 ? 4 + kScaleLoads : 4;
      const char* at = a_rd + (t & 1) * kTileBytes;
      const char* bt = b_rd + (t % 3) * kTileBytes;
      Frags f;
      uint32_t sa[kFM], sb[kFN];
      read(f, at, bt, o, 0);
      if constexpr (Sub == 0) {
        // The group's first use of its scale registers, where the compiler
        // waits for their loads (and, as it does not count the direct-to-LDS
        // loads, for every load of the wave in flight): after this memory
        // phase's reads are issued, while the other group computes.
        take(cur, nxt);
      }
      pick_scales(sa, sb, cur, Sub, 0, lhalf);
#pragma unroll
      for (int i = 0; i < 4; ++i) ld_a(t + 1, i);
      sync<-1, true>();
      compute<0>(acc, f, sa, sb, sel0(Sub, 0), [&](int) {}, [&](int) {});
      sync<-1, false>();
      read(f, at, bt, o, 1);
      if constexpr (kFp4 && !Blocks) pick_scales(sa, sb, cur, Sub, 1, lhalf);
#pragma unroll
      for (int i = 0; i < 4; ++i) ld_b(t + 2, i);
      sync<kWaitM, true>();
      if constexpr (Sub == 0)
        compute<kScaleLoads>(acc, f, sa, sb, sel0(Sub, 1), [&](int) {},
                             [&](int q) { ld_s(nxt, t + kScaleTiles, q); });
      else
        compute<0>(acc, f, sa, sb, sel0(Sub, 1), [&](int) {}, [&](int) {});
      sync<kWaitC, false>();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if (g) barrier();  // group 1 runs one phase behind group 0
    int t = 0;
    for (; t + kScaleTiles <= T; t += kScaleTiles) {
      tile(I0{}, t);
      tile(I1{}, t + 1);
      if constexpr (kScaleTiles == 4) {
        tile(I2{}, t + 2);
        tile(I3{}, t + 3);
      }
    }
    if (t < T) tile(I0{}, t);
    if constexpr (kScaleTiles == 4) {
      if (t + 1 < T) tile(I1{}, t + 1);
      if (t + 2 < T) tile(I2{}, t + 2);
    }
    if (!g) barrier();
    // The scale loads of the last group stay in the program (a load whose
    // result went unused could be removed, and the explicit waits count
    // them), and every load has landed before the epilogue.
    settle(cur);
    settle(nxt);
    wait_vmem();

    if (d_dtype == SG_F32) {
      Base::epilogue(acc, j, nullptr, SG_NONE, D, d_dtype, ldd, lane, g, w4);
    } else {
      // A 16-bit D goes out through LDS: once all waves pass the barrier no
      // fragment read or load is pending, and wave (g, w4) takes 16 KiB of
      // its own.
      barrier();
      char* area = smem + (4 * g + w4) * 16384;
      if (d_dtype == SG_BF16)
        stage_d16<SG_BF16>(acc, area, j.alpha, lane);
      else
        stage_d16<SG_F16>(acc, area, j.alpha, lane);
      const int cc = lane & 7;
      const int nl = 64 * w4 + 8 * cc;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint32_t r = (uint32_t)(8 * s + (lane >> 3));
        const u32x4 d = lds_read16(area, r * 128u + 16u * ((uint32_t)cc ^ (r & 7u)));
        const int ml = 128 * g + (int)r;
        if (ml >= j.m_valid || nl >= j.n_valid) continue;
        uint16_t* p = static_cast<uint16_t*>(D) + (j.d_row0 + ml) * ldd + j.n0 + nl;
        *reinterpret_cast<u32x4*>(p) = d;  // N * 2 is a multiple of 16 bytes
      }
    }
  }

  // The wave's 128 x 64 block of a 16-bit D into `area`: row r (128 bytes),
  // 16-byte chunk c (8 columns) at chunk c XOR (r mod 8), so the 8 rows of
  // a ds_write_b128 phase fill one 128-byte bank line.  Lane l of
  // accumulator block (fm, fn) holds row 32fm + l%32 of the block, columns
  // 32fn + 8q + 4(l/32) .. +3 in registers 4q .. 4q+3; for each pair of q a
  // v_permlane32_swap trades halves between lanes l and l+32, leaving lane l
  // the whole chunk 4fn + 2p + l/32.
  template <int DD>
  __device__ __forceinline__ static void stage_d16(const f32x16 (&acc)[kFM][kFN], char* area,
                                                   float alpha, int lane) {
    const u32x2 none{};
    auto half = [&](int fm, int fn, int q) {
      const f32x4 v = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                       acc[fm][fn][4 * q + 3]};
      return pack_d16<DD>(epi_value<SG_NONE>(v, none, alpha, 0.0f));
    };
    const uint32_t r0 = (uint32_t)(lane & 31), h = (uint32_t)(lane >> 5);
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const u32x2 lo = half(fm, fn, 2 * p), hi = half(fm, fn, 2 * p + 1);
          // lanes 0-31 end with (own lo, partner's lo), lanes 32-63 with
          // (partner's hi, own hi): columns in order either way.
          const auto x = __builtin_amdgcn_permlane32_swap(lo[0], hi[0], false, false);
          const auto y = __builtin_amdgcn_permlane32_swap(lo[1], hi[1], false, false);
          const uint32_t r = 32u * (uint32_t)fm + r0;
          const uint32_t c = 4u * (uint32_t)fn + 2u * (uint32_t)p + h;
          lds_write16(area, r * 128u + 16u * (c ^ (r & 7u)), u32x4{x[0], y[0], x[1], y[1]});
        }
  }
};

// Blocks: p.sf_layout is SG_SF_BLOCKS (else SG_SF_ROWS).
template <int Swz, int Fmt, bool Blocks>
__global__ void __launch_bounds__(512, 1) pingpong_mx_kernel(const MxParams p) {
  using Tile = PingPongMxTile<Swz, Fmt, Blocks>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const ClockStamp cs = clock_begin(p.clk);
  const int total = p.tiles_m * p.tiles_n;
  const int t = xcd_remap(blockIdx.x, total);
  int tm, tn;
  raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int64_t row_bytes = Tile::kFp4 ? p.K / 2 : Tile::kFp6 ? p.K / 4 * 3 : p.K;
  TileJob j;
  j.m_valid = (int)min<int64_t>(256, p.M - m0);
  j.n_valid = (int)min<int64_t>(256, p.N - n0);
  j.a = static_cast<const char*>(p.A) + m0 * row_bytes;
  j.a_pitch = (uint32_t)row_bytes;
  j.a_bytes = (uint32_t)(j.m_valid * row_bytes);
  j.b = static_cast<const char*>(p.B) + n0 * row_bytes;
  j.b_pitch = (uint32_t)row_bytes;
  j.b_bytes = (uint32_t)(j.n_valid * row_bytes);
  // fp6: a shifted row reads 8 bytes past its end at the last K tile.  Below
  // the operand's last tile that is the next tile's first row (in range of
  // the descriptor once it covers 8 more bytes); in the last tile, the rows
  // at the block position of the operand's last row stay unshifted.
  uint32_t ua = 32, ub = 32;
  if (Tile::kFp6) {
    if (p.M - m0 > 256) j.a_bytes += 8;
    else ua = (uint32_t)((p.M - 1 - m0) & 31);
    if (p.N - n0 > 256) j.b_bytes += 8;
    else ub = (uint32_t)((p.N - 1 - n0) & 31);
  }
  j.d_row0 = m0;
  j.n0 = n0;
  j.ldc = 0;
  j.alpha = 1.0f;
  j.beta = 0.0f;
  const SfMap sf = SfMap::make(p.sf_layout, p.K);
  Tile::run(smem, j, sf.tile(p.SFA, m0), sf.tile(p.SFB, n0), sf, p.K, p.D, p.d_dtype, p.N, ua,
            ub);
  clock_end(p.clk, cs);
}

}  // namespace sg
