// pingpong.h -- the 8-wave "ping-pong" mainloop for 256x256 tiles whose A
// and B are both K-major (16-bit elements).
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

#include "gemm_kernels.h"

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
};

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
  // four MFMAs.
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

    if (g) barrier();  // group 1 runs one phase behind group 0
    int bs = 0;        // t mod 3
    for (int t = 0; t < T; ++t) {
      const int as = t & 1, bs2 = bs == 0 ? 2 : bs - 1;  // (t+2) mod 2, (t+2) mod 3
      const char* at = a_rd + as * kTileBytes;
      const char* bt = b_rd + bs * kTileBytes;
      const uint32_t k2 = (uint32_t)(t + 2) * 128u;
      Frags f;
      read(f, at, bt, o, 0);
      end_phase();
      compute(acc, f, lb, rb, b_ring + bs2 * kTileBytes, w4, b_rows, k2, kbytes);
      end_phase();
      read(f, at, bt, o, 1);
      end_phase();
      compute(acc, f, la, ra, a_ring + as * kTileBytes, w4, a_rows, k2, kbytes);
      end_phase();
      bs = bs == 2 ? 0 : bs + 1;
    }
    if (!g) barrier();
    wait_vmem();  // the zero-filled loads past K

    Base::epilogue(acc, j, C, c_dtype, D, d_dtype, ldd, lane, g, w4);
  }
};

template <bool IsBF16, int Swz>
__global__ void __launch_bounds__(512, 1) pingpong_gemm_kernel(const DenseParams p) {
  using Tile = PingPongTile<IsBF16, Swz>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const TileJob j = dense_tile_job<256, 256, false, false>(p, blockIdx.x);
  Tile::run(smem, j, p.K, p.C, p.c_dtype, p.D, p.d_dtype, p.N);
}

template <bool IsBF16, int Swz>
__global__ void __launch_bounds__(512, 1) pingpong_grouped_kernel(const GroupedParams p) {
  using Tile = PingPongTile<IsBF16, Swz>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const TileJob j = grouped_tile_job<256, 256>(p, blockIdx.x);
  Tile::run(smem, j, p.K, nullptr, SG_NONE, p.D, p.d_dtype, p.N);
}

}  // namespace sg
