// deep64.h -- 64x64 tiles with an eight-stage LDS ring, for GEMMs too small
// to give every CU more than one tile (M = N = K = 1024 is 256 such tiles),
// and 128x128 tiles with a five-stage ring, for GEMMs
// with fewer than 256 tiles of 256x256 (M = N = K = 2048 is 256 such tiles).
//
// Why.  Such a tile does 4 MFMAs per wave per 64-wide K tile, a few hundred
// cycles, while a K tile's loads take a load latency (around a microsecond
// from L2) to land.  A double-buffered mainloop therefore waits one latency
// per K tile.  Here the loads run seven K tiles ahead: LDS holds eight
// stages of 16 KiB (A then B, 64 rows x 128 bytes each), and the wait before
// K tile t+1's fragments are read only needs that tile's own loads, issued
// six tiles earlier; the reads of tile t+1 overlap the MFMAs of tile t.
//
// Layout.  A K-major operand uses the XOR map lds_offset<128, 16> and the
// fragment reads of GemmTile.  An MN-major operand is stored as it lies in
// memory, one LDS row per k: for 64x64 tiles 128 bytes (64 m or n values),
// the 16-byte chunks of rows whose bit 1 is set rotated by four chunks; for
// 128x128 tiles 256 bytes, see bmn_offset.  The MFMA
// operand of a lane is 8 consecutive k of one m or n; two transposing reads
// (ds_read_b64_tr_b16) fetch it: in each group of 16 lanes, lane i reads 4
// consecutive m or n of row k0 + i/4, and the read hands lane j the 4 k of
// column j.  One read covers rows k0..k0+3 at 64 bytes each per 32 lanes,
// and the rotation puts those four rows on the four quarters of the banks.
//
// Waves.  Four waves in a 2x2 grid, one (64x64 tiles) or 2x2 (128x128) 32x32
// accumulators each (the GemmTile layout, whose epilogue this tile uses).
// Every wave issues a quarter of a K tile's 1 KiB direct-to-LDS loads; a
// barrier before each K tile makes all of them visible and frees the stage
// the next loads go to.
#pragma once

#include "pingpong.h"

namespace sg {

template <int BM, bool IsBF16, bool AMn, bool BMn>
struct DeepTile {
  static_assert(BM == 64 || BM == 128, "64x64 or 128x128 tiles");
  using Base = GemmTile<BM, BM, IsBF16, AMn, BMn, kSwzDefault, 4>;
  static constexpr int kFM = Base::kFM, kFN = Base::kFN;   // 32x32 blocks per wave
  static constexpr int kStages = BM == 64 ? 8 : 5;
  static constexpr int kBK = 64;
  static constexpr int kOpBytes = BM * 128;                // one operand's K tile
  static constexpr int kStageBytes = 2 * kOpBytes;         // A, then B
  static constexpr int kLdsBytes = kStages * kStageBytes;  // 128 or 160 KiB
  static constexpr int kLoads = 2 * (BM / 32);             // a wave's loads per K tile
  // A wave's loads newer than those of K tile 0 at the first wait, and than
  // those of K tile t+1 in iteration t.
  static constexpr int kFirst = (kStages - 2) * kLoads, kLoop = (kStages - 3) * kLoads;
  static_assert(kFirst == 24 && (kLoop == 20 || kLoop == 16), "vmcnt immediates");

  // Byte offset, in an MN-major operand's stage, of byte `byte` of k-row k.
  // 64x64 tiles: 128-byte rows, rows with bit 1 of k rotated by 64 bytes.
  // 128x128 tiles: 256-byte rows, 32-byte unit u at u XOR 2(k mod 4): one
  // transposing read covers 4 rows x 64 bytes (two units) per 32 lanes,
  // which the key spreads over the 8 units of the bank line.
  static constexpr uint32_t kMnRow = BM * 2;
  __device__ __forceinline__ static uint32_t bmn_offset(uint32_t k, uint32_t byte) {
    if constexpr (BM == 64)
      return k * 128u + ((byte + 64u * ((k >> 1) & 1u)) & 127u);
    else
      return k * 256u + 32u * ((byte >> 5) ^ (2u * (k & 3u))) + (byte & 31u);
  }

  __device__ __forceinline__ static void run(char* smem, const TileJob& j, int64_t K,
                                             const void* C, int c_dtype, void* D,
                                             int d_dtype, int64_t ldd) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lhalf = lane >> 5;

    const u32x4 ra = rsrc_words(j.a, j.a_bytes), rb = rsrc_words(j.b, j.b_bytes);
    const uint32_t kbytes = (uint32_t)K * 2u;
    const int T = (int)((K + kBK - 1) / kBK);
    HalfLoader<kSwzDefault> la, lb;
    la.init(wave, lane, j.a_pitch);
    lb.init(wave, lane, j.b_pitch);
    const uint32_t s0 = lds_addr(smem);

    // Loads of K tile t of one operand into `dst`; past K every chunk is
    // out of range (zero fill).  Regions 4i + wave (1 KiB each).  MN-major:
    // lane l of region r fills k-row 8r + l/8, physical chunk l%8, which
    // holds logical chunk (l%8 + 4 * bit 1 of the row) mod 8.
    auto issue_op = [&](auto mn, const HalfLoader<kSwzDefault>& ld, u32x4 rsrc, uint32_t pitch,
                        int rows_valid, uint32_t dst, int t) {
      if constexpr (!decltype(mn)::value) {
#pragma unroll
        for (int i = 0; i < BM / 32; ++i)
          ld.issue(rsrc, dst, wave, i, rows_valid, (uint32_t)t * 128u, kbytes);
      } else if constexpr (BM == 64) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 4 * i + wave, krow = 8 * r + (lane >> 3);
          const int64_t k = (int64_t)t * kBK + krow;
          const uint32_t c = (uint32_t)((lane & 7) + 4 * ((krow >> 1) & 1)) & 7u;
          const uint32_t off = k < K ? (uint32_t)k * pitch + 16u * c : kOutOfRange;
          dma16(rsrc, off, dst + (uint32_t)r * 1024u);
        }
      } else {
        // 128x128: region r holds k-rows 4r .. 4r+3; lane l fills physical
        // bytes 16(l%16) of row 4r + l/16, which hold the logical bytes the
        // (self-inverse) unit XOR maps there.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * i + wave, krow = 4 * r + (lane >> 4);
          const int64_t k = (int64_t)t * kBK + krow;
          const uint32_t lb = bmn_offset((uint32_t)krow, 16u * (uint32_t)(lane & 15)) -
                              (uint32_t)krow * kMnRow;
          const uint32_t off = k < K ? (uint32_t)k * pitch + lb : kOutOfRange;
          dma16(rsrc, off, dst + (uint32_t)r * 1024u);
        }
      }
    };
    // K tile t into stage t mod kStages.
    auto issue = [&](int t) {
      const uint32_t stage = s0 + (uint32_t)(t % kStages) * kStageBytes;
      issue_op(std::integral_constant<bool, AMn>{}, la, ra, j.a_pitch, j.m_valid, stage, t);
      issue_op(std::integral_constant<bool, BMn>{}, lb, rb, j.b_pitch, j.n_valid,
               stage + kOpBytes, t);
    };

    const typename Base::FragOffsets o = Base::frag_offsets(wm, wn, lrow, lhalf);
    f32x16 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int k = 0; k < kFN; ++k) acc[i][k] = f32x16{};

    // The fragments of one K tile: four 16-wide steps of A and B.
    struct Frags {
      u32x4 a[kBK / 16][kFM], b[kBK / 16][kFN];
    };
    // An MN-major operand's fragment for columns col0 .. col0+31 (m or n):
    // lane l gets k = 16 kk + 8 (l/32) + e (e = 0..7) of column col0 + l%32.
    // Lane group G = l/16 covers columns col0 + 16 (G%2) + 0..15 and, for
    // read r, k0 = 16 kk + 8 (G/2) + 4r; its lane i supplies row k0 + i/4,
    // columns +4 (i%4) .. +3, and receives the 4 k of its own column.
    const int tr_g = lane >> 4, tr_i = lane & 15;
    auto gather = [&](const char* base, int col0, int kk) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
      const uint32_t c2 = 2u * (uint32_t)(col0 + 16 * (tr_g & 1) + 4 * (tr_i & 3));
      u32x4 v;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t k = (uint32_t)(16 * kk + 8 * (tr_g >> 1) + 4 * r + (tr_i >> 2));
        const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)((__attribute__((address_space(3))) char*)base + bmn_offset(k, c2)));
        const u32x2 w = __builtin_bit_cast(u32x2, t);
        v[2 * r] = w[0];
        v[2 * r + 1] = w[1];
      }
      return v;
    };
    auto read = [&](Frags& f, int t) {
      const char* as = smem + (t % kStages) * kStageBytes;
      const char* bs = as + kOpBytes;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
        for (int fm = 0; fm < kFM; ++fm) {
          if constexpr (!AMn)
            f.a[kk][fm] = lds_read16(as, o.a[kk] + fm * 32 * 128);
          else
            f.a[kk][fm] = gather(as, wm * 32 * kFM + 32 * fm, kk);
        }
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn) {
          if constexpr (!BMn)
            f.b[kk][fn] = lds_read16(bs, o.b[kk] + fn * 32 * 128);
          else
            f.b[kk][fn] = gather(bs, wn * 32 * kFN + 32 * fn, kk);
        }
      }
    };

#pragma unroll
    for (int t = 0; t < kStages - 1; ++t) issue(t);

    // Software pipelined: the fragments of K tile t+1 are read while the
    // MFMAs of tile t run.  Before iteration t the wave waits for its loads
    // of tile t+1 (the kLoop newer ones may stay in flight); the barrier
    // makes every wave's loads of t+1 visible and frees the stage of tile
    // t-1, whose fragments were read in iteration t-2, for the loads of tile
    // t + kStages - 1.
    Frags f0, f1;
    asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    PingPongTile<IsBF16, kSwzDefault>::barrier();
    read(f0, 0);
    // The reads of K step kk of tile t.
    auto read_kk = [&](Frags& f, int t, int kk) {
      const char* as = smem + (t % kStages) * kStageBytes;
      const char* bs = as + kOpBytes;
#pragma unroll
      for (int fm = 0; fm < kFM; ++fm) {
        if constexpr (!AMn)
          f.a[kk][fm] = lds_read16(as, o.a[kk] + fm * 32 * 128);
        else
          f.a[kk][fm] = gather(as, wm * 32 * kFM + 32 * fm, kk);
      }
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) {
        if constexpr (!BMn)
          f.b[kk][fn] = lds_read16(bs, o.b[kk] + fn * 32 * 128);
        else
          f.b[kk][fn] = gather(bs, wn * 32 * kFN + 32 * fn, kk);
      }
    };
    // 64x64: each 16-wide K step's MFMA over `cur` comes first and the reads
    // of the same step of tile t+1 after it, so the MFMAs start right after
    // the barrier; the loads of tile t + kStages - 1 follow the first step
    // (measured 2.6% faster at 1024^3 than loads, then reads, then MFMAs).
    // 128x128 (four MFMAs a step): the loads, then all the reads, then the
    // MFMAs (the other order measured 8-16% slower at 1536^3 and 2048^3).
    // `steps`: the 16-wide K steps of the tile that hold any of K (4 but in
    // the last tile), so no MFMA multiplies only the zero fill past K.
    auto iteration = [&](int t, Frags& cur, Frags& nxt, int steps) {
      if constexpr (kLoop == 20)
        asm volatile("s_waitcnt vmcnt(20) lgkmcnt(0)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
      PingPongTile<IsBF16, kSwzDefault>::barrier();
      if constexpr (BM != 64) {
        issue(t + kStages - 1);
        read(nxt, t + 1);  // past the last tile: stale LDS, never used
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
          if (kk >= steps) break;
#pragma unroll
          for (int m = 0; m < kFM * kFN; ++m) {
            const int fm = m / kFN, fn = (fm & 1) ? kFN - 1 - m % kFN : m % kFN;
            acc[fm][fn] = mfma32x32x16<IsBF16>(cur.b[kk][fn], cur.a[kk][fm], acc[fm][fn]);
          }
        }
        return;
      }
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        if (kk < steps) {
#pragma unroll
          for (int m = 0; m < kFM * kFN; ++m) {
            // snake order: consecutive MFMAs share an operand
            const int fm = m / kFN, fn = (fm & 1) ? kFN - 1 - m % kFN : m % kFN;
            acc[fm][fn] = mfma32x32x16<IsBF16>(cur.b[kk][fn], cur.a[kk][fm], acc[fm][fn]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        read_kk(nxt, t + 1, kk);  // past the last tile: stale LDS, never used
        __builtin_amdgcn_sched_barrier(0);
        if (kk == 0) issue(t + kStages - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int last_steps = (int)((K - (int64_t)(T - 1) * kBK + 15) / 16);  // 1..4 (T > 0)
    int t = 0;
    for (; t + 2 < T; t += 2) {
      iteration(t, f0, f1, kBK / 16);
      iteration(t + 1, f1, f0, kBK / 16);
    }
    if (t + 1 < T) {
      iteration(t, f0, f1, kBK / 16);
      iteration(t + 1, f1, f0, last_steps);
    } else if (t < T) {
      iteration(t, f0, f1, last_steps);
    }
    wait_vmem();  // the loads past K

    if (d_dtype == SG_F32 && C == nullptr) {
      PingPongTile<IsBF16, kSwzDefault>::barrier();  // every wave's reads are done
      store_f32_via_lds(acc, j, smem + wave * kWaveBytes, D, ldd, lane, wm, wn);
    } else {
      Base::epilogue(acc, j, C, c_dtype, D, d_dtype, ldd, lane, wm, wn);
    }
  }

  // An fp32 D (no C) through LDS.  Lane l of accumulator block (fm, fn) holds
  // row 32fm + l%32 of the wave's block, columns 32fn + 8q + 4(l/32) .. +3 in
  // registers 4q .. 4q+3: 16-byte chunk 8fn + 2q + l/32 of a kRowBytes row.
  // The wave writes its block into its own area, chunk c of row r at chunk
  // c XOR (r mod 8), which gives the 8 rows of one ds_write_b128 phase (8
  // lanes, one 128-byte bank line) 8 distinct places in the line, then
  // reads it back one contiguous KiB per instruction
  // and stores whole rows: kRowBytes / 16 lanes per row, where the register
  // layout gave each store instruction 32 bytes per row.
  static constexpr int kRowBytes = 128 * kFN;                 // fp32 row of a wave
  static constexpr int kWaveBytes = 32 * kFM * kRowBytes;     // 4 or 16 KiB
  static_assert(4 * kWaveBytes <= kLdsBytes, "staging fits the ring");
  __device__ __forceinline__ static uint32_t row_key(uint32_t r) { return r & 7u; }
  __device__ __forceinline__ static void store_f32_via_lds(const f32x16 (&acc)[kFM][kFN],
                                                           const TileJob& j, char* area,
                                                           void* D, int64_t ldd, int lane,
                                                           int wm, int wn) {
    const u32x2 none{};
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = epi_value<SG_NONE>(
              f32x4{acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                    acc[fm][fn][4 * q + 3]},
              none, j.alpha, 0.0f);
          const uint32_t r = (uint32_t)(32 * fm + (lane & 31));
          const uint32_t c = (uint32_t)(8 * fn + 2 * q + (lane >> 5));
          lds_write16(area, r * kRowBytes + 16u * (c ^ row_key(r)), __builtin_bit_cast(u32x4, v));
        }
    constexpr int kLanesPerRow = kRowBytes / 16, kRowsPerStep = 64 / kLanesPerRow;
    const uint32_t cc = (uint32_t)(lane % kLanesPerRow);
    const int nl = wn * Base::kWN + 4 * (int)cc;
#pragma unroll
    for (int s = 0; s < kWaveBytes / 1024; ++s) {
      const uint32_t r = (uint32_t)(kRowsPerStep * s + lane / kLanesPerRow);
      const u32x4 d = lds_read16(area, r * kRowBytes + 16u * (cc ^ row_key(r)));
      const int ml = wm * Base::kWM + (int)r;
      if (ml >= j.m_valid || nl >= j.n_valid) continue;
      *reinterpret_cast<u32x4*>(static_cast<float*>(D) + (j.d_row0 + ml) * ldd + j.n0 + nl) = d;
    }
  }
};

template <int BM, bool IsBF16, bool AMn, bool BMn>
__global__ void __launch_bounds__(256, 1) deep_gemm_kernel(const DenseParams p) {
  using Tile = DeepTile<BM, IsBF16, AMn, BMn>;
  __shared__ __attribute__((aligned(4096))) char smem[Tile::kLdsBytes];
  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = dense_tile_job<BM, BM, AMn, BMn>(p, blockIdx.x);
  Tile::run(smem, j, p.K, p.C, p.c_dtype, p.D, p.d_dtype, p.ldd);
  clock_end(p.clk, cs);
}

}  // namespace sg
