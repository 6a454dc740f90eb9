// pingpong16.h -- the 8-wave ping-pong mainloop (pingpong.h) computed with
// v_mfma_f32_16x16x32 instead of v_mfma_f32_32x32x16.
//
// Why.  The GEMM runs at the clock its power allows, and the power depends on
// the data.  Measured on MI355X with random operands and the MFMA pipe 96%
// busy, 16x16x32 MFMAs hold 2.37 GHz where 32x32x16 MFMAs of the same FLOPs
// drop to 2.08 GHz.  A 16x16x32 MFMA takes 16 cycles, so one wave per SIMD
// cannot issue its fragment reads and loads between them; the ping-pong's
// second wave per SIMD does that work.
//
// The roles, phases and LDS rings are those of pingpong.h.  Wave w4 of group
// g owns output rows [128g, +128) and columns [64 w4, +64) as 8x4 blocks of
// 16x16 accumulators (128 accumulator registers).  A phase covers 32 of K:
// 12 fragment reads (lane l: row l%16 of a 16-row block, 16-byte chunk 4kh +
// l/16 of the row, conflict-free under the swizzle), or 32 MFMAs.  For K a
// multiple of 64 the memory phases also issue the group's loads (A of tile
// t+1 in the first of tile t, B of tile t+2 in the second), so the compute
// phases are MFMAs only: a direct-to-LDS load among a wave's MFMAs delays its
// next MFMA by about 7 cycles even with m0 written ahead, while a memory
// phase has room to spare (measured: 2-3% faster than issuing them between
// the MFMAs, 4% slower with all eight in the first memory phase).  Otherwise
// each compute phase issues the four loads of a half tile, one per eight
// MFMAs, as in pingpong.h.
//
// The epilogue goes through LDS: a 16-bit C arrives with the loads of the
// last two K tiles (which would otherwise fetch zeros past K), and a 16-bit
// D is staged there and stored as whole 128-byte row segments.
#pragma once

#include "pingpong.h"

namespace sg {

// AMn / BMn: A is [K][M] / B is [K][N] (MN-major); such an operand's half
// tiles hold one 256-byte row per k (mn256_lds_offset) and its fragments
// come from transposing reads.  Only for K a multiple of 64 with at least
// two K tiles.  OutSwz: whether the epilogue's C and D staging in LDS use
// their XOR keys (the library) or the logical chunk order (the output half
// of the layout ablation); Swz is the operands' layout.
template <bool IsBF16, int Swz, bool AMn = false, bool BMn = false, bool OutSwz = true>
struct PingPong16Tile {
  using PP = PingPongTile<IsBF16, Swz>;
  static constexpr int kHalfBytes = PP::kHalfBytes;
  static constexpr int kTileBytes = PP::kTileBytes;
  static constexpr int kBK = PP::kBK;
  static constexpr int kARing = PP::kARing, kBRing = PP::kBRing;
  static constexpr int kLdsBytes = PP::kLdsBytes;  // 160 KiB
  static constexpr int kI = 8, kJ = 4;              // 16x16 blocks per wave (M, N)

  // Fragments of one 32-wide K half of a tile.
  struct Frags {
    u32x4 a[kI], b[kJ];
  };

  // Per-lane byte offsets inside an operand's K tile: [K half][block
  // parity]; block 2p+q is 4096 p bytes past entry q (blocks 32 rows apart
  // share the XOR key).
  struct Offsets {
    uint32_t a[2][2], b[2][2];
    uint32_t bt[kJ];  // MN-major B: block j, K half 0, read 0 (see read)
    uint32_t at[kI];  // MN-major A: block i, the same
  };

  __device__ __forceinline__ static Offsets offsets(int g, int w4, int lane) {
    const int r = lane & 15, c = lane >> 4;
    Offsets o;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        o.a[kh][q] = g * kHalfBytes + lds_offset<128, Swz>(16 * q + r, 4 * kh + c);
        o.b[kh][q] = (w4 >> 1) * kHalfBytes +
                     lds_offset<128, Swz>((w4 & 1) * 64 + 16 * q + r, 4 * kh + c);
      }
    if constexpr (BMn) {
      // Lane group c = l/16 takes k rows 8c + 4r + 32kh .. +3 (read r, K half
      // kh), lane r = l%16 supplies row (l%16)/4 of them at columns
      // 64(w4%2) + 16j + 4(l%4) of its half; the key is the same for every r
      // and kh (they add 4r + 32kh to k).
#pragma unroll
      for (int jb = 0; jb < kJ; ++jb)
        o.bt[jb] = (w4 >> 1) * kHalfBytes +
                   mn256_lds_offset((uint32_t)(8 * c + (r >> 2)),
                                    2u * (uint32_t)(64 * (w4 & 1) + 16 * jb + 4 * (r & 3)));
    }
    if constexpr (AMn) {  // the group's own half, all 128 m
#pragma unroll
      for (int ib = 0; ib < kI; ++ib)
        o.at[ib] = g * kHalfBytes + mn256_lds_offset((uint32_t)(8 * c + (r >> 2)),
                                                     2u * (uint32_t)(16 * ib + 4 * (r & 3)));
    }
    return o;
  }

  // Two transposing reads give lane l the 8 k (32kh + 8(l/16) .. +7) of the
  // column l%16 of block j: in each 16-lane group, lane i reads 4 columns of
  // one k row and receives the 4 k of its own column.
  __device__ __forceinline__ static u32x4 read_bt(const char* bt, uint32_t off) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    typedef __attribute__((address_space(3))) char lds_char;
    const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)bt + off));
    const v4i16 t1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)bt + off + 1024u));
    const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
    return u32x4{w0[0], w0[1], w1[0], w1[1]};
  }

  // The K-exact loader of an MN-major half (group g: columns 128g .. +128
  // of the tile): load q of wave w4 fills region 4q + w4 with k rows 4(4q +
  // w4) .. +3, lane l taking row l/16 and the 16 bytes whose place is
  // 16(l%16) (the unit XOR is its own inverse); columns past the tile read
  // as zero.  The K position (64 rows a tile) travels in the SGPR offset.
  __device__ __forceinline__ static void init_bmn(KExactHalfLoader<Swz>& x, int g, int w4,
                                                  int lane, uint32_t pitch, int cols) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k = (uint32_t)(4 * (4 * q + w4) + (lane >> 4));
      const uint32_t lbyte = mn256_lds_offset(k, 16u * (uint32_t)(lane & 15)) - k * 256u;
      const int col = (int)(lbyte >> 1);
      x.voff[q] = col < cols ? k * pitch + 2u * (uint32_t)(128 * g + col) : kOutOfRange;
    }
  }

  __device__ __forceinline__ static void read(Frags& f, const char* at, const char* bt,
                                              const Offsets& o, int kh) {
#pragma unroll
    for (int i = 0; i < kI; ++i) {
      if constexpr (AMn)
        f.a[i] = read_bt(at, o.at[i] + 8192u * (uint32_t)kh);
      else
        f.a[i] = lds_read16(at, o.a[kh][i & 1] + (i >> 1) * 4096);
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if constexpr (BMn)
        f.b[j] = read_bt(bt, o.bt[j] + 8192u * (uint32_t)kh);
      else
        f.b[j] = lds_read16(bt, o.b[kh][j & 1] + (j >> 1) * 4096);
    }
  }

  // 32 MFMAs with the four loads of one half tile between them, one per
  // eight MFMAs (without the MFMAs for a wave whose output rows are all past
  // M: it still loads its share and keeps the barriers).  MFMA rows take B
  // rows (n), columns take A rows (m).  The blocks go in snake order (row i
  // of blocks left to right, row i+1 right to left), so consecutive MFMAs
  // always share an operand: measured 1.5-2% more clock at the power limit
  // than restarting each row at block 0.
  template <bool Active>
  __device__ __forceinline__ static void compute(f32x4 (&acc)[kI][kJ], const Frags& f,
                                                 const HalfLoader<Swz>& ld, u32x4 rsrc,
                                                 uint32_t half, int w4, int rows_valid,
                                                 uint32_t kbyte0, uint32_t kbytes) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int mm = 8 * q + m, i = mm >> 2, j = (i & 1) ? 3 - (mm & 3) : (mm & 3);
        if (Active && m == 7) {  // the load's m0 write, one MFMA ahead (set_m0)
          __builtin_amdgcn_sched_barrier(0);
          ld.prep(half, w4, q);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (Active) acc[i][j] = mfma16x16x32<IsBF16>(f.b[j], f.a[i], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (Active)
        ld.go(rsrc, q, rows_valid, kbyte0, kbytes);
      else
        ld.issue(rsrc, half, w4, q, rows_valid, kbyte0, kbytes);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The same with the K-exact loader, whose m0 write goes one MFMA ahead of
  // its load (set_m0) when the wave has MFMAs to put between them.
  template <bool Active>
  __device__ __forceinline__ static void compute_x(f32x4 (&acc)[kI][kJ], const Frags& f,
                                                   const KExactHalfLoader<Swz>& ld, u32x4 rsrc,
                                                   uint32_t half, int w4, uint32_t kbyte0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int mm = 8 * q + m, i = mm >> 2, j = (i & 1) ? 3 - (mm & 3) : (mm & 3);
        if (Active && m == 7) {
          __builtin_amdgcn_sched_barrier(0);
          if (q == 0) ld.template prep<0>(half, w4);
          if (q == 1) ld.template prep<1>(half, w4);
          if (q == 2) ld.template prep<2>(half, w4);
          if (q == 3) ld.template prep<3>(half, w4);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (Active) acc[i][j] = mfma16x16x32<IsBF16>(f.b[j], f.a[i], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (Active) {
        if (q == 0) ld.template go<0>(rsrc, kbyte0);
        if (q == 1) ld.template go<1>(rsrc, kbyte0);
        if (q == 2) ld.template go<2>(rsrc, kbyte0);
        if (q == 3) ld.template go<3>(rsrc, kbyte0);
      } else {  // no MFMA between an m0 write and its load: the joint form
        if (q == 0) ld.template issue<0>(rsrc, half, w4, kbyte0);
        if (q == 1) ld.template issue<1>(rsrc, half, w4, kbyte0);
        if (q == 2) ld.template issue<2>(rsrc, half, w4, kbyte0);
        if (q == 3) ld.template issue<3>(rsrc, half, w4, kbyte0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // 32 MFMAs over one K half's fragments and nothing else (snake order, see
  // compute).
  template <bool Active>
  __device__ __forceinline__ static void mfmas(f32x4 (&acc)[kI][kJ], const Frags& f) {
    if constexpr (Active) {
#pragma unroll
      for (int mm = 0; mm < 32; ++mm) {
        const int i = mm >> 2, j = (i & 1) ? 3 - (mm & 3) : (mm & 3);
        acc[i][j] = mfma16x16x32<IsBF16>(f.b[j], f.a[i], acc[i][j]);
      }
    }
  }

  // The four loads of one half tile (from a memory phase, where the joint
  // m0 write costs nothing that matters).
  __device__ __forceinline__ static void load_half(const KExactHalfLoader<Swz>& ld, u32x4 rsrc,
                                                   uint32_t half, int w4, uint32_t kbyte0) {
    ld.template issue<0>(rsrc, half, w4, kbyte0);
    ld.template issue<1>(rsrc, half, w4, kbyte0);
    ld.template issue<2>(rsrc, half, w4, kbyte0);
    ld.template issue<3>(rsrc, half, w4, kbyte0);
  }

  // The waits that end the four phases of a K tile, then the barrier.
  template <int Phase>
  __device__ __forceinline__ static void sync() {
    if constexpr (Phase == 0)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else if constexpr (Phase == 2)
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    else if constexpr (Phase == 3)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    PP::barrier();
  }

  // One K tile t of the K-exact mainloop.  Its memory phases issue the
  // group's loads, so the compute phases are MFMAs only:
  //   memory  (K half 0): reads the fragments, then loads A of tile t+1 into
  //           A slot (t+1) mod 2 (group g's half: its four waves were done
  //           with tile t-1 there by the last barrier) and B of tile t+2 into
  //           B slot (t+2) mod 3 (both groups were done with tile t-1 there);
  //   compute (K half 0);
  //   memory  (K half 1): reads; then all but the wave's newest 8 loads have
  //           landed (the other group's B of tile t+1, for this group's
  //           next read);
  //   compute (K half 1; the last tile also loads the C block's fourth
  //           quarter, into A slot t mod 2); then all but the newest 4 loads
  //           have landed (the wave's own A of tile t+1).
  // `xa`, `rat`, `ka`: the loader, descriptor and SGPR offset of A(t+1);
  // `xb`, `rbt`, `kb` those of B(t+2); `xq`, `rq` the fourth C quarter.
  template <bool Active, bool LastQ3>
  __device__ __forceinline__ static void ktile(
      f32x4 (&acc)[kI][kJ], int t, int bs, const KExactHalfLoader<Swz>& xa, u32x4 rat,
      uint32_t ka, const KExactHalfLoader<Swz>& xb, u32x4 rbt, uint32_t kb,
      const KExactHalfLoader<Swz>& xq, u32x4 rq, uint32_t a_ring, uint32_t b_ring,
      const char* a_rd, const char* b_rd, const Offsets& o, int w4) {
    const int as = t & 1, bs2 = bs == 0 ? 2 : bs - 1;  // t mod 2, (t+2) mod 3
    const char* at = a_rd + as * kTileBytes;
    const char* bt = b_rd + bs * kTileBytes;
    Frags f;
    if constexpr (Active) read(f, at, bt, o, 0);
    load_half(xa, rat, a_ring + (as ^ 1) * kTileBytes, w4, ka);
    sync<0>();
    mfmas<Active>(acc, f);
    sync<1>();
    if constexpr (Active) read(f, at, bt, o, 1);
    load_half(xb, rbt, b_ring + bs2 * kTileBytes, w4, kb);
    sync<2>();
    if constexpr (LastQ3)
      compute_x<Active>(acc, f, xq, rq, a_ring + as * kTileBytes, w4, 0u);
    else
      mfmas<Active>(acc, f);
    sync<3>();
  }

  // Where the last two K tiles' loads put a 16-bit C.  Those loads would
  // fetch the zero tiles T and T+1; instead, wave w4 of group g brings the C
  // block of its own outputs (128 rows x 64 columns, 16 KiB) into the four
  // half slots they fill, quarter Q (rows 32Q..32Q+31 of the block) into B
  // slot T mod 3, A slot T mod 2, B slot (T+1) mod 3, A slot (T+1) mod 2 for
  // Q = 0..3, half g, laid out by cblock_lds_offset: load q of the quarter
  // fills region 4q + w4 with rows 32Q + 8q .. +7, lane l taking row l / 8
  // of them and the chunk whose place is l mod 8.
  struct CBlock {
    u32x4 rsrc;      // C from row d_row0 + 128g, column n0 of the tile
    uint32_t pitch;  // bytes per C row
    int rows;        // C rows of the block that exist
    int lrow;        // this lane's row inside a 1 KiB region (0..7)
    uint32_t col[4]; // this lane's byte offset in a row, for region 4q + w4

    __device__ __forceinline__ void init(const TileJob& j, const void* C, int g, int w4,
                                         int lane) {
      const int64_t row0 = j.d_row0 + 128 * g;
      rows = min(j.m_valid - 128 * g, 128);
      pitch = (uint32_t)j.ldc * 2u;
      // Records up to the 16-byte chunk holding the tile's last valid element
      // of its last valid row (the base is 16-byte aligned, so that chunk
      // never crosses a page C does not touch); chunks past it read as zero.
      const uint32_t bytes =
          rows > 0 ? (uint32_t)(rows - 1) * pitch + (((uint32_t)j.n_valid * 2u + 15u) & ~15u)
                   : 0u;
      rsrc = rsrc_words(static_cast<const char*>(C) + (row0 * j.ldc + j.n0) * 2, bytes);
      lrow = lane >> 3;
#pragma unroll
      for (int q = 0; q < 4; ++q)  // (the key of row 32Q + r is that of r)
        col[q] = 128u * (uint32_t)w4 +
                 16u * ((uint32_t)(lane & 7) ^
                        (OutSwz ? cblock_key((uint32_t)(8 * q + lrow)) : 0u));
    }
    // The loader of quarter Q: rows past the block read as zero.
    __device__ __forceinline__ KExactHalfLoader<Swz> quarter(int Q) const {
      KExactHalfLoader<Swz> x;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * Q + 8 * q + lrow;
        x.voff[q] = r < rows ? (uint32_t)r * pitch + col[q] : kOutOfRange;
      }
      return x;
    }
  };

  // Mainloop for K a multiple of 64 (the prologue has loaded B of tiles 0
  // and 1 and A of tile 0).  Loads past the operand go through the empty
  // descriptors `ra0`, `rb0` (zero fill) or, with LdsC (T >= 2), bring the
  // wave's C block: quarter 0 as B of tile T, 1 as A of tile T, 2 as B of
  // tile T+1, 3 in the last compute phase into A slot (T-1) mod 2.
  template <bool Active, bool LdsC>
  __device__ __forceinline__ static void mainloop_x(
      f32x4 (&acc)[kI][kJ], const KExactHalfLoader<Swz>& la, const KExactHalfLoader<Swz>& lb,
      u32x4 ra, u32x4 rb, u32x4 ra0, u32x4 rb0, uint32_t a_ring, uint32_t b_ring,
      const char* a_rd, const char* b_rd, const Offsets& o, int g, int w4, int T,
      const TileJob& j, const void* C, int lane, uint32_t kstep_a, uint32_t kstep_b) {
    if (g) PP::barrier();  // group 1 runs one phase behind group 0
    int bs = 0;            // t mod 3
    int t = 0;
    for (; t + 2 < T; ++t) {
      ktile<Active, false>(acc, t, bs, la, ra, (uint32_t)(t + 1) * kstep_a, lb, rb,
                           (uint32_t)(t + 2) * kstep_b, la, ra0, a_ring, b_ring, a_rd, b_rd, o,
                           w4);
      bs = bs == 2 ? 0 : bs + 1;
    }
    if constexpr (LdsC) {
      CBlock cb;
      cb.init(j, C, g, w4, lane);
      ktile<Active, false>(acc, t, bs, la, ra, (uint32_t)(t + 1) * kstep_a, cb.quarter(0),
                           cb.rsrc, 0u, la, ra0, a_ring, b_ring, a_rd, b_rd, o, w4);
      bs = bs == 2 ? 0 : bs + 1;
      ktile<Active, true>(acc, t + 1, bs, cb.quarter(1), cb.rsrc, 0u, cb.quarter(2), cb.rsrc,
                          0u, cb.quarter(3), cb.rsrc, a_ring, b_ring, a_rd, b_rd, o, w4);
    } else {
      for (; t < T; ++t) {
        const u32x4 rat = t + 1 < T ? ra : ra0;
        ktile<Active, false>(acc, t, bs, la, rat, (uint32_t)(t + 1) * kstep_a, lb, rb0,
                             (uint32_t)(t + 2) * kstep_b, la, ra0, a_ring, b_ring, a_rd, b_rd,
                             o, w4);
        bs = bs == 2 ? 0 : bs + 1;
      }
    }
    if (!g) PP::barrier();
  }

  // The epilogue through the wave's C block area (cblock_lds_offset): lane l
  // of accumulator block (i, jn) holds row 16i + l%16 of the block, columns
  // 16jn + 4(l/16) .. +3, i.e. half (l/16) mod 2 of chunk 2jn + l/32.  A
  // 16-bit C (CD) is read from there; a 16-bit D is staged in the same
  // regions (dstage_offset) and stored a whole 128-byte row segment per 8
  // lanes (row 8s + l/8, chunk l%8), 16 stores of 16 bytes instead of 32 of
  // 8.  An fp32 D is stored from registers.
  template <int CD, int DD>
  __device__ __forceinline__ static void epilogue_lds_t(const f32x4 (&acc)[kI][kJ],
                                                        const TileJob& j, char* const (&cq)[4],
                                                        void* D, int64_t ldd, int lane, int g,
                                                        int w4) {
    auto place = [&](int i, int jn) {
      const uint32_t r = (uint32_t)(16 * i + (lane & 15));
      const uint32_t off =
          cblock_lds_offset((uint32_t)w4, r, (uint32_t)(2 * jn + (lane >> 5)), OutSwz);
      return (off & 16383u) + 8u * (uint32_t)((lane >> 4) & 1);
    };
    u32x2 c[kI][kJ];
    if constexpr (CD != SG_NONE) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int jn = 0; jn < kJ; ++jn) c[i][jn] = lds_read8(cq[i >> 1], place(i, jn));
    }
    if constexpr (DD == SG_F32) {
#pragma unroll
      for (int i = 0; i < kI; ++i) {
        const int ml = 128 * g + 16 * i + (lane & 15);
        if (ml >= j.m_valid) continue;
        const int64_t row = (j.d_row0 + ml) * ldd + j.n0;
#pragma unroll
        for (int jn = 0; jn < kJ; ++jn) {
          const int nl = 64 * w4 + 16 * jn + 4 * (lane >> 4);
          if (nl >= j.n_valid) continue;
          store_d_chunk<CD, DD>(acc[i][jn], c[i][jn], D, row + nl, j.alpha, j.beta);
        }
      }
    } else {
      // Lane l holds 4 columns of row 16i + l%16: with ρ = l/16, columns
      // 16jn + 4ρ .. +3.  For each pair of blocks (2jp, 2jp+1) a
      // v_permlane16_swap trades them between lane rows ρ = 0, 1 and ρ = 2,
      // 3, leaving lane l the whole 16-byte chunk 2(2jp + ρ%2) + ρ/2 of the
      // row (columns in order), written to dstage_offset with
      // ds_write_b128.  A wave's LDS accesses complete in order: the writes
      // follow every read of C, the row reads follow the writes.
      const int rho = lane >> 4;
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int jp = 0; jp < kJ / 2; ++jp) {
          const u32x2 x0 = pack_d16<DD>(epi_value<CD>(acc[i][2 * jp], c[i][2 * jp], j.alpha,
                                                      j.beta));
          const u32x2 x1 = pack_d16<DD>(epi_value<CD>(acc[i][2 * jp + 1], c[i][2 * jp + 1],
                                                      j.alpha, j.beta));
          const auto a = __builtin_amdgcn_permlane16_swap(x0[0], x1[0], false, false);
          const auto b = __builtin_amdgcn_permlane16_swap(x0[1], x1[1], false, false);
          const uint32_t r = (uint32_t)(16 * i + (lane & 15));
          const uint32_t ch = (uint32_t)(4 * jp + 2 * (rho & 1) + (rho >> 1));
          lds_write16(cq[i >> 1], dstage_offset<OutSwz>((uint32_t)w4, r, ch),
                      u32x4{a[0], b[0], a[1], b[1]});
        }
      store_d16_block<OutSwz>(cq, j, D, ldd, lane, g, w4);
    }
  }

  // cd: the C type in LDS, SG_NONE for none.  Takes 16-bit C or 16-bit D.
  __device__ __forceinline__ static void epilogue_lds(const f32x4 (&acc)[kI][kJ],
                                                      const TileJob& j, char* const (&cq)[4],
                                                      int cd, void* D, int d_dtype, int64_t ldd,
                                                      int lane, int g, int w4) {
#define SG_EPI(CD, DD) return epilogue_lds_t<CD, DD>(acc, j, cq, D, ldd, lane, g, w4)
    if (d_dtype == SG_F32) {
      if (cd == SG_BF16) SG_EPI(SG_BF16, SG_F32);
      SG_EPI(SG_F16, SG_F32);
    }
    if (d_dtype == SG_BF16) {
      if (cd == SG_BF16) SG_EPI(SG_BF16, SG_BF16);
      if (cd == SG_F16) SG_EPI(SG_F16, SG_BF16);
      SG_EPI(SG_NONE, SG_BF16);
    }
    if (cd == SG_BF16) SG_EPI(SG_BF16, SG_F16);
    if (cd == SG_F16) SG_EPI(SG_F16, SG_F16);
    SG_EPI(SG_NONE, SG_F16);
#undef SG_EPI
  }

  template <bool Active>
  __device__ __forceinline__ static void mainloop(f32x4 (&acc)[kI][kJ],
                                                  const HalfLoader<Swz>& la,
                                                  const HalfLoader<Swz>& lb, u32x4 ra, u32x4 rb,
                                                  int a_rows, int b_rows, uint32_t a_ring,
                                                  uint32_t b_ring, const char* a_rd,
                                                  const char* b_rd, const Offsets& o, int g,
                                                  int w4, int T, uint32_t kbytes) {
    if (g) PP::barrier();  // group 1 runs one phase behind group 0
    int bs = 0;            // t mod 3
    for (int t = 0; t < T; ++t) {
      const int as = t & 1, bs2 = bs == 0 ? 2 : bs - 1;  // (t+2) mod 2, (t+2) mod 3
      const char* at = a_rd + as * kTileBytes;
      const char* bt = b_rd + bs * kTileBytes;
      const uint32_t k2 = (uint32_t)(t + 2) * 128u;
      Frags f;
      if constexpr (Active) read(f, at, bt, o, 0);
      PP::end_phase();
      compute<Active>(acc, f, lb, rb, b_ring + bs2 * kTileBytes, w4, b_rows, k2, kbytes);
      PP::end_phase();
      if constexpr (Active) read(f, at, bt, o, 1);
      PP::end_phase();
      compute<Active>(acc, f, la, ra, a_ring + as * kTileBytes, w4, a_rows, k2, kbytes);
      PP::end_phase();
      bs = bs == 2 ? 0 : bs + 1;
    }
    if (!g) PP::barrier();
  }

  // Mainloop and epilogue of one tile; `smem` is the 160 KiB of LDS.
  __device__ __forceinline__ static void run(char* smem, const TileJob& j, int64_t K,
                                             const void* C, int c_dtype, void* D,
                                             int d_dtype, int64_t ldd) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, w4 = wave & 3;

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
    // Bytes of B's descriptor per K tile: 64 k of a K-major row, or 64 rows
    // of an MN-major B.
    const uint32_t kstep_a = AMn ? 64u * j.a_pitch : 128u;
    const uint32_t kstep_b = BMn ? 64u * j.b_pitch : 128u;
    KExactHalfLoader<Swz> xam, xbm;
    if constexpr (AMn) init_bmn(xam, g, w4, lane, j.a_pitch, a_rows);
    if constexpr (BMn) init_bmn(xbm, g, w4, lane, j.b_pitch, b_rows);

    // Tiles 0 and 1 (B before A, the order the mainloop keeps); the K-exact
    // mainloop loads A of tile 1 itself.
    const bool kexact = AMn || BMn || (K & (kBK - 1)) == 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (BMn) {
        xbm.template issue<0>(rb, b_ring + t * kTileBytes, w4, t * kstep_b);
        xbm.template issue<1>(rb, b_ring + t * kTileBytes, w4, t * kstep_b);
        xbm.template issue<2>(rb, b_ring + t * kTileBytes, w4, t * kstep_b);
        xbm.template issue<3>(rb, b_ring + t * kTileBytes, w4, t * kstep_b);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          lb.issue(rb, b_ring + t * kTileBytes, w4, i, b_rows, t * 128u, kbytes);
      }
      if (t == 1 && kexact) break;
      if constexpr (AMn) {
        xam.template issue<0>(ra, a_ring + t * kTileBytes, w4, t * kstep_a);
        xam.template issue<1>(ra, a_ring + t * kTileBytes, w4, t * kstep_a);
        xam.template issue<2>(ra, a_ring + t * kTileBytes, w4, t * kstep_a);
        xam.template issue<3>(ra, a_ring + t * kTileBytes, w4, t * kstep_a);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          la.issue(ra, a_ring + t * kTileBytes, w4, i, a_rows, t * 128u, kbytes);
      }
    }
    if (kexact) {  // tile 0 has landed; B of tile 1 may still be in flight
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
      PP::barrier();
    } else {
      PP::end_phase();
    }

    const Offsets o = offsets(g, w4, lane);
    f32x4 acc[kI][kJ];
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int k = 0; k < kJ; ++k) acc[i][k] = f32x4{};

    // A wave whose 128 output rows all lie past M (the second group of a tile
    // with at most 128 valid rows) runs the mainloop without its MFMAs.
    // A 16-bit C comes in through the last two K tiles' loads when K is a
    // multiple of 64 and 128 C rows stay within 32-bit buffer offsets.
    const bool ldsc = kexact && T >= 2 && C != nullptr &&
                      (c_dtype == SG_BF16 || c_dtype == SG_F16) && j.ldc <= (int64_t{1} << 22);
    if (kexact) {
      KExactHalfLoader<Swz> xa, xb;
      if constexpr (AMn)
        xa = xam;
      else
        xa.init(la, a_rows);
      if constexpr (BMn)
        xb = xbm;
      else
        xb.init(lb, b_rows);
      const u32x4 ra0 = rsrc_words(j.a, 0), rb0 = rsrc_words(j.b, 0);
      if (a_rows > 0 && ldsc)
        mainloop_x<true, true>(acc, xa, xb, ra, rb, ra0, rb0, a_ring, b_ring, a_rd, b_rd, o, g,
                               w4, T, j, C, lane, kstep_a, kstep_b);
      else if (a_rows > 0)
        mainloop_x<true, false>(acc, xa, xb, ra, rb, ra0, rb0, a_ring, b_ring, a_rd, b_rd, o, g,
                                w4, T, j, C, lane, kstep_a, kstep_b);
      else
        mainloop_x<false, false>(acc, xa, xb, ra, rb, ra0, rb0, a_ring, b_ring, a_rd, b_rd, o,
                                 g, w4, T, j, C, lane, kstep_a, kstep_b);
    } else if (a_rows > 0) {
      mainloop<true>(acc, la, lb, ra, rb, a_rows, b_rows, a_ring, b_ring, a_rd, b_rd, o, g, w4,
                     T, kbytes);
    } else {
      mainloop<false>(acc, la, lb, ra, rb, a_rows, b_rows, a_ring, b_ring, a_rd, b_rd, o, g,
                      w4, T, kbytes);
    }
    wait_vmem();  // the C block, or the zero-filled loads past K

    // Through LDS: a 16-bit C that came in with the last loads, and a 16-bit
    // D.  Every fragment read is done once all waves pass the barrier, and
    // the wave's C block area is written by its own loads only.
    const bool d16 = d_dtype == SG_BF16 || d_dtype == SG_F16;
    if (ldsc || (d16 && C == nullptr)) {
      PP::barrier();
      char* cq[4];
      cblock_quarters(cq, smem, T, g, kTileBytes, kHalfBytes);
      if (a_rows > 0)
        epilogue_lds(acc, j, cq, ldsc ? c_dtype : SG_NONE, D, d_dtype, ldd, lane, g, w4);
    } else {
      epilogue16<kI, kJ>(acc, j, C, c_dtype, D, d_dtype, ldd, lane, 128 * g, 64 * w4);
    }
  }
};

template <bool IsBF16, int Swz, bool AMn = false, bool BMn = false, bool OutSwz = true>
__global__ void __launch_bounds__(512, 1) pingpong16_gemm_kernel(const DenseParams p) {
  using Tile = PingPong16Tile<IsBF16, Swz, AMn, BMn, OutSwz>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = dense_tile_job<256, 256, AMn, BMn>(p, blockIdx.x);
  Tile::run(smem, j, p.K, p.C, p.c_dtype, p.D, p.d_dtype, p.ldd);
  clock_end(p.clk, cs);
}

template <bool IsBF16, int Swz>
__global__ void __launch_bounds__(512, 1) pingpong16_grouped_kernel(const GroupedParams p) {
  using Tile = PingPong16Tile<IsBF16, Swz>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = grouped_tile_job<256, 256>(p, blockIdx.x);
  Tile::run(smem, j, p.K, nullptr, SG_NONE, p.D, p.d_dtype, p.N);
  clock_end(p.clk, cs);
}

}  // namespace sg
