// mx_kernels.h -- block-scaled (MXFP8) GEMM kernel template.
//
// D[m][n] = sum_blk 2^(SFA[m][blk]-127) 2^(SFB[n][blk]-127)
//           * sum_{k in blk} A[m][k] B[n][k]            (32-element blocks)
// -- output (m, n) takes SFA for row m and SFB for column n of the block
// ("06 Blackwell Tensor Core - tcgen05 MMA", section "Block-Scaled MMA").
//
// Same tile machinery as the 16-bit kernels: e4m3 operands staged K-major in
// LDS, 128 bytes (= 128 elements = 4 scale blocks) of K per stage, under the
// same swizzle.  Operand and scale layout of v_mfma_scale_f32_32x32x64_
// f8f6f4 (checked on the GPU with one-hot operands): lane l supplies row l%32
// and, of the 64-wide K step, K values [16h, 16h+16) in its low 16 bytes and
// [32+16h, 32+16h+16) in its high 16 bytes (h = l/32); the e8m0 byte of lane
// l scales 32-element block h of the step for row l%32 -- so block 0 is the
// low halves of both lane halves and block 1 the high halves.  The scales are
// not staged: each lane loads the 4 scale bytes of its row for the current
// stage straight into a VGPR.
#pragma once

#include "gemm_device.h"
#include "gemm_kernels.h"

namespace sg {

struct MxParams {
  const void* A;    // e4m3 [M][K]
  const void* SFA;  // e8m0 [M][K/32] (SG_SF_ROWS) or in 64-row blocks (SG_SF_BLOCKS)
  const void* B;    // e4m3 [N][K]
  const void* SFB;  // e8m0 [N][K/32] or in 64-row blocks
  void* D;
  int64_t M, N, K;
  int d_dtype;
  int sf_layout;    // SG_SF_ROWS or SG_SF_BLOCKS
  int tiles_m, tiles_n;
  int group_m;
  ClockTrace clk;
};

// Where the scale byte of 32-element block b of row r lies, relative to a
// tile's first row (tile rows start at multiples of 64).
//   SG_SF_ROWS:   e8m0 [rows][K/32]: byte r * (K/32) + b.
//   SG_SF_BLOCKS: the bytes of 64 rows x 16 blocks together: 1 KiB for rows
//                 [64i, 64i+64) and blocks [16g, 16g+16), row r's 16 bytes
//                 at 16 (r mod 64), the even blocks of the group first
//                 (block b at 8 (b mod 2) + (b mod 16) / 2); blocks (i, g)
//                 in the order i * G + g, G = ceil(K/512) groups a row.  A
//                 load of one group's bytes for 32 or 64 consecutive rows
//                 reads contiguous bytes (4 or 8 cache lines); in the rows
//                 layout the same load touches a line per row.  The lane
//                 halves of the scaled MFMA scale the even and the odd
//                 blocks of a step: each finds its bytes in one 8-byte half.
struct SfMap {
  uint32_t blocked, pitch, groups;

  __device__ __forceinline__ static SfMap make(int layout, int64_t K) {
    return SfMap{layout == SG_SF_BLOCKS ? 1u : 0u, (uint32_t)(K / 32),
                 (uint32_t)((K / 32 + 15) / 16)};
  }
  // The part of the offset that depends on the row.
  __device__ __forceinline__ uint32_t row(uint32_t r) const {
    return blocked ? (r >> 6) * groups * 1024u + (r & 63u) * 16u : r * pitch;
  }
  // The part that depends on the block index b (uniform in a wave).
  __device__ __forceinline__ uint32_t block(uint32_t b) const {
    return blocked ? (b >> 4) * 1024u + in_unit(b) : b;
  }
  // Block layout: block b's byte inside its row's 16 bytes.
  __device__ __forceinline__ static uint32_t in_unit(uint32_t b) {
    return 8u * (b & 1u) + ((b & 15u) >> 1);
  }
  __device__ __forceinline__ const char* tile(const void* sf, int64_t row0) const {
    const char* p = static_cast<const char*>(sf);
    return blocked ? p + (row0 >> 6) * (int64_t)groups * 1024 : p + row0 * (int64_t)pitch;
  }
  // Bytes from a tile's first row to the end of its rows_valid rows.
  __device__ __forceinline__ uint32_t tile_bytes(int rows_valid) const {
    return blocked ? (uint32_t)((rows_valid + 63) / 64) * groups * 1024u
                   : (uint32_t)rows_valid * pitch;
  }
};

__device__ __forceinline__ f32x16 mfma_scale_f8(const u32x4 (&a)[2],
                                                const u32x4 (&b)[2], f32x16 c,
                                                uint32_t sa, uint32_t sb,
                                                int kk) {
  const i32x8 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                    (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
  const i32x8 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                    (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
  // Format codes 0/0: both operands OCP fp8 E4M3.  The op-select immediate
  // picks byte 2*kk of the scale register (see MxTile::spread).
  if (kk == 0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0,
                                                           (int)sa, 0, (int)sb);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 2,
                                                         (int)sa, 2, (int)sb);
}

template <int BM, int BN, int Swz>
struct MxTile {
  static constexpr int kBK = 128;           // fp8 elements (= bytes) per stage
  static constexpr int kRowBytes = 128;
  static constexpr int kATileBytes = BM * kRowBytes;
  static constexpr int kBTileBytes = BN * kRowBytes;
  static constexpr int kStageBytes = kATileBytes + kBTileBytes;
  static constexpr int kWM = BM / 2, kWN = BN / 2;
  static constexpr int kFM = kWM / 32, kFN = kWN / 32;
  static_assert(kStageBytes % 4096 == 0, "stage bases must keep the swizzle phase");

  struct Scales {
    uint32_t a[kFM], b[kFN];
  };

  // Rows layout: one dword = the 4 scale bytes of K blocks [4kt, 4kt+4) of
  // a row.  Block layout: the 2 bytes of blocks 4kt + h and 4kt + 2 + h
  // (h = l/32: the lane's half of the row's 16 bytes).  `spread` then puts
  // the lane's block of step kk at byte 2kk, where op-select 2kk reads it.
  __device__ __forceinline__ static void load_scales(
      Scales& s, __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
      const SfMap& sf, int kt, int lane, int wm, int wn, int m_valid,
      int n_valid) {
    const int lrow = lane & 31;
    const uint32_t b = 4u * (uint32_t)kt + (uint32_t)(lane >> 5);
    const uint32_t kb = sf.blocked ? sf.block(b) : sf.block(4u * (uint32_t)kt);
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm) {
      const int r = wm * kWM + fm * 32 + lrow;
      const uint32_t off = r < m_valid ? sf.row((uint32_t)r) + kb : kOutOfRange;
      s.a[fm] = sf.blocked ? buffer_load2(rsa, off) : buffer_load4(rsa, off);
    }
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn) {
      const int r = wn * kWN + fn * 32 + lrow;
      const uint32_t off = r < n_valid ? sf.row((uint32_t)r) + kb : kOutOfRange;
      s.b[fn] = sf.blocked ? buffer_load2(rsb, off) : buffer_load4(rsb, off);
    }
  }

  // The v_perm selector of `spread`: rows layout, bytes h and 2 + h of the
  // dword to bytes 0 and 2; block layout, bytes 0 and 1 (selector 12 gives
  // a zero byte).
  __device__ __forceinline__ static uint32_t spread_sel(const SfMap& sf, int lane) {
    const uint32_t h = (uint32_t)(lane >> 5);
    return sf.blocked ? 0x0c010c00u : 0x0c000c00u | h | ((2u + h) << 16);
  }
  __device__ __forceinline__ static uint32_t spread(uint32_t v, uint32_t sel) {
    return __builtin_amdgcn_perm(0u, v, sel);
  }

  struct Frags {
    u32x4 a[kFM][2], b[kFN][2];
  };

  // Lane half h = l/32 supplies 16-byte chunk 4*kk + h (block 2*kk) then
  // chunk 4*kk + 2 + h (block 2*kk + 1).
  __device__ __forceinline__ static void read_frags(Frags& f, const char* As,
                                                    const char* Bs, int wm, int wn,
                                                    int lrow, int lhalf, int kk) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.a[fm][h] = lds_read16(As, lds_offset<kRowBytes, Swz>(
                                        wm * kWM + fm * 32 + lrow, 4 * kk + 2 * h + lhalf));
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.b[fn][h] = lds_read16(Bs, lds_offset<kRowBytes, Swz>(
                                        wn * kWN + fn * 32 + lrow, 4 * kk + 2 * h + lhalf));
  }

  __device__ __forceinline__ static void mfmas(f32x16 (&acc)[kFM][kFN], const Frags& f,
                                               const uint32_t (&sa)[kFM],
                                               const uint32_t (&sb)[kFN], int kk) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
        acc[fm][fn] = mfma_scale_f8(f.b[fn], f.a[fm], acc[fm][fn], sb[fn], sa[fm], kk);
  }

  static constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

  // One 64-wide K step: the next step's 2*(kFM+kFN) fragment reads are
  // interleaved with this step's MFMAs, with `Vmem` loads of the next K tile
  // spread over the same stretch.
  template <int Vmem>
  __device__ __forceinline__ static void step(f32x16 (&acc)[kFM][kFN], const Frags& cur,
                                              Frags& nxt, const char* As, const char* Bs,
                                              int wm, int wn, int lrow, int lhalf,
                                              int kk_next, const uint32_t (&sa)[kFM],
                                              const uint32_t (&sb)[kFN], int kk) {
    read_frags(nxt, As, Bs, wm, wn, lrow, lhalf, kk_next);
    mfmas(acc, cur, sa, sb, kk);
    constexpr int kReads = 2 * (kFM + kFN), kMfma = kFM * kFN;
    constexpr int kPer = kMfma / kReads > 0 ? kMfma / kReads : 1;
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if constexpr (Vmem > 0)
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (Vmem + kReads - 1) / kReads, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPer, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // One K tile of 128: compute on stage `cur` while tile kt+1 (operands by
  // direct-to-LDS DMA into `nxt`, scales into VGPRs) loads.  Same barrier
  // placement and distinct-stage-object rule as the 16-bit kernels.
  __device__ __forceinline__ static void k_tile(
      f32x16 (&acc)[kFM][kFN], Frags& f0, Frags& f1,
      OperandLoader<BM, false, Swz, 1>& la, OperandLoader<BN, false, Swz, 1>& lb,
      Scales& sc, Scales& sc_next, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
      __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb, const SfMap& sf, char* cur,
      char* nxt, const TileJob& j, int tid, int lane, int wm, int wn, int lrow, int lhalf,
      int kt, int kt_total, int Ki) {
    constexpr int kVmem = BM / 32 + BN / 32;
    // Unconditional loads (same basic block as the MFMAs they interleave
    // with); after the last tile they start at k = K and only zero-fill
    // `nxt`, and the scale loads re-read the last tile's scales.
    const bool more = kt + 1 < kt_total;
    const int k1 = more ? (kt + 1) * kBK : Ki;
    la.issue(ra, nxt, tid, j.m_valid, k1, Ki);
    lb.issue(rb, nxt + kATileBytes, tid, j.n_valid, k1, Ki);
    load_scales(sc_next, rsa, rsb, sf, more ? kt + 1 : kt, lane, wm, wn, j.m_valid,
                j.n_valid);
    uint32_t sa[kFM], sb[kFN];
    const uint32_t sel = spread_sel(sf, lane);
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm) sa[fm] = spread(sc.a[fm], sel);
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn) sb[fn] = spread(sc.b[fn], sel);
    step<kVmem>(acc, f0, f1, cur, cur + kATileBytes, wm, wn, lrow, lhalf, 1, sa, sb, 0);
    wait_vmem();
    __syncthreads();
    // Unconditional (see the 16-bit kernels): after the last tile the reads
    // of `nxt` are stale and unused.
    step<0>(acc, f1, f0, nxt, nxt + kATileBytes, wm, wn, lrow, lhalf, 0, sa, sb, 1);
    sc = sc_next;
  }

  __device__ __forceinline__ static void run(char* s0, char* s1, const TileJob& j,
                                             const char* sfa, const char* sfb,
                                             const SfMap& sf, int64_t K, void* D,
                                             int d_dtype, int64_t ldd) {
    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; readfirstlane lets the
    // compiler keep it (and every LDS base derived from it) in SGPRs.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, lhalf = lane >> 5;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(j.a, j.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(j.b, j.b_bytes);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sfa, sf.tile_bytes(j.m_valid));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sfb, sf.tile_bytes(j.n_valid));

    f32x16 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int k = 0; k < kFN; ++k) acc[i][k] = f32x16{};

    const int Ki = (int)K;
    const int kt_total = Ki / kBK;
    OperandLoader<BM, false, Swz, 1> la;
    OperandLoader<BN, false, Swz, 1> lb;
    la.init(tid, j.a_pitch);
    lb.init(tid, j.b_pitch);
    Scales sc, sc_next;
    if (kt_total > 0) {
      la.issue(ra, s0, tid, j.m_valid, 0, Ki);
      lb.issue(rb, s0 + kATileBytes, tid, j.n_valid, 0, Ki);
      load_scales(sc, rsa, rsb, sf, 0, lane, wm, wn, j.m_valid, j.n_valid);
    }
    wait_vmem();
    __syncthreads();

    Frags f0, f1;
    if (kt_total > 0) read_frags(f0, s0, s0 + kATileBytes, wm, wn, lrow, lhalf, 0);

    // Two K tiles per trip (fixed stage objects), odd last tile peeled.
    int kt = 0;
    for (; kt + 1 < kt_total; kt += 2) {
      k_tile(acc, f0, f1, la, lb, sc, sc_next, ra, rb, rsa, rsb, sf, s0, s1, j, tid,
             lane, wm, wn, lrow, lhalf, kt, kt_total, Ki);
      k_tile(acc, f0, f1, la, lb, sc, sc_next, ra, rb, rsa, rsb, sf, s1, s0, j, tid,
             lane, wm, wn, lrow, lhalf, kt + 1, kt_total, Ki);
    }
    if (kt < kt_total)
      k_tile(acc, f0, f1, la, lb, sc, sc_next, ra, rb, rsa, rsb, sf, s0, s1, j, tid,
             lane, wm, wn, lrow, lhalf, kt, kt_total, Ki);

    GemmTile<BM, BN, true, false, false, Swz>::epilogue(acc, j, nullptr, SG_NONE, D,
                                                        d_dtype, ldd, lane, wm, wn);
  }
};

template <int BM, int BN, int Swz>
__global__ void __launch_bounds__(kThreads, 1) mx_gemm_kernel(const MxParams p) {
  using Tile = MxTile<BM, BN, Swz>;
  __shared__ __attribute__((aligned(4096))) char s0[Tile::kStageBytes];
  __shared__ __attribute__((aligned(4096))) char s1[Tile::kStageBytes];

  const ClockStamp cs = clock_begin(p.clk);
  const int total = p.tiles_m * p.tiles_n;
  const int t = xcd_remap(blockIdx.x, total);
  int tm, tn;
  raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  TileJob j;
  j.m_valid = (int)min<int64_t>(BM, p.M - m0);
  j.n_valid = (int)min<int64_t>(BN, p.N - n0);
  j.a = static_cast<const char*>(p.A) + m0 * p.K;
  j.a_pitch = (uint32_t)p.K;
  j.a_bytes = (uint32_t)(j.m_valid * p.K);
  j.b = static_cast<const char*>(p.B) + n0 * p.K;
  j.b_pitch = (uint32_t)p.K;
  j.b_bytes = (uint32_t)(j.n_valid * p.K);
  j.d_row0 = m0;
  j.n0 = n0;
  j.ldc = 0;
  j.alpha = 1.0f;
  j.beta = 0.0f;
  const SfMap sf = SfMap::make(p.sf_layout, p.K);
  Tile::run(s0, s1, j, sf.tile(p.SFA, m0), sf.tile(p.SFB, n0), sf, p.K, p.D, p.d_dtype, p.N);
  clock_end(p.clk, cs);
}

}  // namespace sg
