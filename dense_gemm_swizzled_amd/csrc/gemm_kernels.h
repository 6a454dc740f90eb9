// gemm_kernels.h -- the dense / grouped swizzled GEMM kernel template and
// its launch parameters (included by the per-dtype translation units).
//
// Structure of one workgroup (256 threads = 4 wave64s, one output tile):
//   1. tile schedule: workgroup id -> (group, tile row, tile column), with an
//      XCD-aware remap and GROUP_M-style rasterisation (the Triton matmul
//      listing in "Tensor Cores, layouts, and swizzling" groups tile rows
//      for cache reuse; here each of the 8 XCDs, which have private L2s, is
//      given a contiguous range of that order);
//   2. global -> LDS: each lane moves 16 bytes per load, consecutive lanes
//      consecutive chunks of a row (the cooperative loader of "LBO, SBO and
//      SWZ for a tcgen05 tile", section 2); the global order stays logical
//      and only the LDS destination is swizzled (same page, section 3);
//   3. a two-stage LDS ring: the loads for K tile k+1 are in flight while
//      tile k is consumed; one barrier per K tile keeps a stage from being
//      overwritten before every wave has read it (the rule of the Hopper
//      mainloop in "Tensor Cores, layouts, and swizzling");
//   4. MFMA: each wave owns a (BM/2) x (BN/2) block of 32x32 fp32
//      accumulators, fed by ds_read_b128 of swizzled 16-byte chunks; the
//      first K step starts from zero (the accumulate-flag rule of "06
//      Blackwell Tensor Core", section "How tcgen05.mma Executes");
//   5. epilogue: registers -> global with optional C, no LDS staging (the
//      Results of "Swizzling explained properly" measure no gain from
//      swizzling the output tile).
#pragma once

#include <type_traits>

#include "gemm_device.h"
#include "../../include/swizzled_gemm.h"

namespace sg {

struct DenseParams {
  const void* A;
  const void* B;
  const void* C;
  void* D;
  int64_t M, N, K;
  int64_t lda, ldb, ldc, ldd;  // leading dimensions in elements
  float alpha, beta;           // D = alpha * A.B + beta * C
  int c_dtype, d_dtype;
  int tiles_m, tiles_n;
  int group_m;
  ClockTrace clk;
};

struct GroupedParams {
  const void* A;
  const void* B;
  void* D;
  int64_t N, K;
  int d_dtype;
  int G;
  int tiles_n;
  int group_m;
  ClockTrace clk;
  int64_t m_off[SG_MAX_GROUPS + 1];      // row offsets of the groups
  int32_t tile_start[SG_MAX_GROUPS + 1]; // first tile id of each group
};

// Spread workgroups so that each XCD (workgroups are dealt to the 8 XCDs
// round robin) receives a contiguous range of tile ids.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = wg & 7, idx = wg >> 3;
  return x * per + (x < rem ? x : rem) + idx;
}

// Tile id -> (tile row, tile column): columns of group_m tile rows.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n,
                                       int group_m, int& tm, int& tn) {
  const int width = group_m * tiles_n;
  const int g = t / width;
  const int first = g * group_m;
  const int gm = min(tiles_m - first, group_m);
  const int local = t - g * width;
  tm = first + local % gm;
  tn = local / gm;
}

// Where one workgroup's operand panels and output tile live.
struct TileJob {
  const char* a;        // A panel base (see loaders for the addressing)
  uint32_t a_bytes;     // bytes readable from a
  uint32_t a_pitch;     // bytes per source row of A
  int m_valid;          // rows of this tile that exist (<= BM)
  const char* b;
  uint32_t b_bytes;
  uint32_t b_pitch;
  int n_valid;
  int64_t d_row0;       // first output row (absolute)
  int64_t n0;           // first output column
  int64_t ldc;          // leading dimension of C in elements
  float alpha, beta;    // D = alpha * acc + beta * C
};

// Epilogue element work shared by every kernel.  One chunk is 4 consecutive
// n of one output row: C as loaded (f32x4 for fp32, u32x2 for 16-bit), then
// D = acc + C in fp32, rounded to D's type (round to nearest even).
template <int CD>
using c_chunk_t = typename std::conditional<CD == SG_F32, f32x4, u32x2>::type;

template <int CD>
__device__ __forceinline__ c_chunk_t<CD> load_c_chunk(const void* C, int64_t idx) {
  if constexpr (CD == SG_F32)
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(C) + idx);
  else
    return *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(C) + idx);
}

// alpha * acc + beta * C of one chunk, in fp32.
template <int CD>
__device__ __forceinline__ f32x4 epi_value(f32x4 v, const c_chunk_t<CD>& c, float alpha,
                                           float beta) {
  if constexpr (CD != SG_NONE) {
    f32x4 cf;
    if constexpr (CD == SG_F32) {
      cf = c;
    } else if constexpr (CD == SG_BF16) {
      cf = f32x4{bf16_to_f32(c[0] & 0xffffu), bf16_to_f32(c[0] >> 16),
                 bf16_to_f32(c[1] & 0xffffu), bf16_to_f32(c[1] >> 16)};
    } else {
      cf = f32x4{f16_to_f32(c[0] & 0xffffu), f16_to_f32(c[0] >> 16),
                 f16_to_f32(c[1] & 0xffffu), f16_to_f32(c[1] >> 16)};
    }
    // alpha * acc + (beta * c), one rounding each; with alpha = beta = 1
    // this is the single fp32 add acc + c.
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(alpha, v[e], beta * cf[e]);
  } else {
    v *= alpha;
  }
  return v;
}

// A chunk rounded to a 16-bit D type (round to nearest even).
template <int DD>
__device__ __forceinline__ u32x2 pack_d16(f32x4 v) {
  static_assert(DD == SG_BF16 || DD == SG_F16, "16-bit D");
  if constexpr (DD == SG_BF16)
    return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  else
    return u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
}

template <int CD, int DD>
__device__ __forceinline__ void store_d_chunk(f32x4 v, const c_chunk_t<CD>& c, void* D,
                                              int64_t idx, float alpha, float beta) {
  v = epi_value<CD>(v, c, alpha, beta);
  if constexpr (DD == SG_F32)
    *reinterpret_cast<f32x4*>(static_cast<float*>(D) + idx) = v;
  else
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(D) + idx) = pack_d16<DD>(v);
}

// Epilogue of a wave's NI x NJ blocks of 16x16 accumulators (v_mfma_f32_
// 16x16x32 with B rows as MFMA rows): lane l of block (i, jn) holds output
// row mw + 16i + l%16 and columns nw + 16jn + 4(l/16) .. +3 of the tile.  C
// of the next block row is loaded before the current one is stored; C
// addresses are clamped into the valid rectangle, stores are masked.
template <int NJ, int CD>
__device__ __forceinline__ void load_c_row16(c_chunk_t<CD> (&c)[NJ], const TileJob& j,
                                             const void* C, int64_t ldd, int lane, int mw,
                                             int nw, int i) {
  if constexpr (CD != SG_NONE) {
    const int ml = min(mw + 16 * i + (lane & 15), j.m_valid - 1);
    const int64_t base = (j.d_row0 + ml) * j.ldc + j.n0;
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) {
      const int nl = min(nw + 16 * jn + 4 * (lane >> 4), j.n_valid - 4);
      c[jn] = load_c_chunk<CD>(C, base + nl);
    }
  }
}

template <int NI, int NJ, int CD, int DD>
__device__ __forceinline__ void epilogue16_t(const f32x4 (&acc)[NI][NJ], const TileJob& j,
                                             const void* C, void* D, int64_t ldd, int lane,
                                             int mw, int nw) {
  // C is loaded a group of kG block rows at a time, the next group before
  // the current one is stored: all of the wave's C at once when it fits in
  // 64 registers (16-bit C of 8x4 blocks), else groups of 32 registers.
  constexpr int kRegs = CD == SG_F32 ? 4 : 2;  // registers per chunk
  constexpr int kAll = NI * NJ * kRegs <= 64;
  constexpr int kG0 = 32 / (NJ * kRegs);
  constexpr int kG = kAll ? NI : (kG0 < 1 ? 1 : kG0);
  c_chunk_t<CD> cb[2][kG][NJ];
#pragma unroll
  for (int i = 0; i < kG; ++i) load_c_row16<NJ, CD>(cb[0][i], j, C, ldd, lane, mw, nw, i);
#pragma unroll
  for (int g0 = 0; g0 < NI; g0 += kG) {
    if (g0 + kG < NI) {
#pragma unroll
      for (int i = 0; i < kG; ++i)
        load_c_row16<NJ, CD>(cb[((g0 / kG) + 1) & 1][i], j, C, ldd, lane, mw, nw, g0 + kG + i);
    }
#pragma unroll
    for (int ii = 0; ii < kG; ++ii) {
      const int i = g0 + ii;
      const int ml = mw + 16 * i + (lane & 15);
      if (ml >= j.m_valid) continue;
      const int64_t row = (j.d_row0 + ml) * ldd + j.n0;
#pragma unroll
      for (int jn = 0; jn < NJ; ++jn) {
        const int nl = nw + 16 * jn + 4 * (lane >> 4);
        if (nl >= j.n_valid) continue;
        store_d_chunk<CD, DD>(acc[i][jn], cb[(g0 / kG) & 1][ii][jn], D, row + nl, j.alpha,
                              j.beta);
      }
    }
  }
}

// The same with the element types chosen at run time.
template <int NI, int NJ>
__device__ __forceinline__ void epilogue16(const f32x4 (&acc)[NI][NJ], const TileJob& j,
                                           const void* C, int c_dtype, void* D, int d_dtype,
                                           int64_t ldd, int lane, int mw, int nw) {
#define SG_EPI(CD, DD) return epilogue16_t<NI, NJ, CD, DD>(acc, j, C, D, ldd, lane, mw, nw)
  if (d_dtype == SG_F32) {
    if (c_dtype == SG_F32) SG_EPI(SG_F32, SG_F32);
    if (c_dtype == SG_BF16) SG_EPI(SG_BF16, SG_F32);
    if (c_dtype == SG_F16) SG_EPI(SG_F16, SG_F32);
    SG_EPI(SG_NONE, SG_F32);
  }
  if (d_dtype == SG_BF16) {
    if (c_dtype == SG_F32) SG_EPI(SG_F32, SG_BF16);
    if (c_dtype == SG_BF16) SG_EPI(SG_BF16, SG_BF16);
    if (c_dtype == SG_F16) SG_EPI(SG_F16, SG_BF16);
    SG_EPI(SG_NONE, SG_BF16);
  }
  if (c_dtype == SG_F32) SG_EPI(SG_F32, SG_F16);
  if (c_dtype == SG_BF16) SG_EPI(SG_BF16, SG_F16);
  if (c_dtype == SG_F16) SG_EPI(SG_F16, SG_F16);
  SG_EPI(SG_NONE, SG_F16);
#undef SG_EPI
}

// Waves = 4: one wave per SIMD, each wave owns a (BM/2) x (BN/2) block.
// Waves = 8: two waves per SIMD (the hardware interleaves them, and twice as
// many waves issue the direct-to-LDS loads), each owning (BM/2) x (BN/4).
template <int BM, int BN, bool IsBF16, bool AMn, bool BMn, int Swz, int Waves = 4>
struct GemmTile {
  static constexpr int kBK = 64;            // K elements per stage
  static constexpr int kRowBytes = 128;     // kBK * 2 bytes
  static constexpr int kRowStride = lds_row_stride<kRowBytes, Swz>();  // 144 when padded
  static constexpr int kATileBytes = BM * kRowStride;
  static constexpr int kBTileBytes = BN * kRowStride;
  static constexpr int kStageBytes = kATileBytes + kBTileBytes;
  static constexpr int kWavesN = Waves / 2;         // waves along N (2 along M)
  static constexpr int kWM = BM / 2, kWN = BN / kWavesN;  // per-wave block
  static constexpr int kFM = kWM / 32, kFN = kWN / 32;
  static_assert(kStageBytes % 4096 == 0 || Swz == kSwzPad,
                "stage bases must keep the swizzle phase");
  static_assert(kFM >= 1 && kFN >= 1, "each wave needs at least one 32x32 block");

  using ALoader = OperandLoader<BM, AMn, Swz, 2, Waves>;
  using BLoader = OperandLoader<BN, BMn, Swz, 2, Waves>;

  // Fragments of one 16-wide K step: lane l holds row l%32 of each 32-row
  // fragment and K chunk 2*kk + l/32.
  struct Frags {
    u32x4 a[kFM], b[kFN];
  };

  // Per-lane LDS byte offsets of fragment 0 for each 16-wide K step.  Rows
  // 32 apart share the XOR key (it depends on the row only through the bank
  // line index modulo 16, i.e. row/2 mod 16, or row mod 8 for 128-byte
  // lines), so fragment f sits exactly f * 32 row strides further (the
  // padded layout is linear): a constant the ds_read offset field absorbs.
  struct FragOffsets {
    uint32_t a[kBK / 16], b[kBK / 16];
  };

  __device__ __forceinline__ static FragOffsets frag_offsets(int wm, int wn, int lrow,
                                                             int lhalf) {
    FragOffsets o;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      o.a[kk] = lds_offset<kRowBytes, Swz>(wm * kWM + lrow, 2 * kk + lhalf);
      o.b[kk] = lds_offset<kRowBytes, Swz>(wn * kWN + lrow, 2 * kk + lhalf);
    }
    return o;
  }

  __device__ __forceinline__ static void read_frags(Frags& f, const char* As,
                                                    const char* Bs, const FragOffsets& o,
                                                    int kk) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
      f.a[fm] = lds_read16(As, o.a[kk] + fm * 32 * kRowStride);
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn)
      f.b[fn] = lds_read16(Bs, o.b[kk] + fn * 32 * kRowStride);
  }

  // MFMA rows take B rows (n), columns take A rows (m): each lane then ends
  // up holding 4 consecutive n of one m (wide epilogue stores).
  __device__ __forceinline__ static void mfmas(f32x16 (&acc)[kFM][kFN], const Frags& f) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
        acc[fm][fn] = mfma32x32x16<IsBF16>(f.b[fn], f.a[fm], acc[fm][fn]);
  }

  // Instruction-scheduling hints (LLVM AMDGPU sched_group_barrier masks).
  static constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

  // One 16-wide K step: the next step's fragment reads (kFM + kFN ds_reads)
  // are interleaved one per two MFMAs of this step, and `vmem` buffer loads
  // of the next K tile are spread over the same stretch, so that the wave's
  // LDS and global traffic issues in the shadow of the matrix core.
  template <int Vmem>
  __device__ __forceinline__ static void step(f32x16 (&acc)[kFM][kFN], const Frags& cur,
                                              Frags& nxt, const char* As, const char* Bs,
                                              const FragOffsets& o, int kk) {
    read_frags(nxt, As, Bs, o, kk);
    mfmas(acc, cur);
    constexpr int kReads = kFM + kFN, kMfma = kFM * kFN;
    constexpr int kPerRead = kMfma / kReads;
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if constexpr (Vmem > 0)
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (Vmem + kReads - 1) / kReads, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPerRead, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Loads of the next K tile issued during 16-wide K step `kk` (1..3).  With
  // one wave per SIMD the tile's direct-to-LDS loads are spread over the
  // three steps that run before the barrier (issuing them all in one step
  // stalls the wave on a full load queue and drains the MFMA pipe).  With two
  // waves per SIMD each wave has half as many loads and the other wave keeps
  // the matrix core busy, so they go out at the start of the tile, which
  // gives them the most time to land (measured faster at 8192^3).
  template <int Loader, int KK>
  struct Share {
    static constexpr int kA = ALoader::kIssues, kB = BLoader::kIssues;
    static constexpr int kTotal = kA + kB;
    static constexpr int kSpread = Waves == 8 ? 1 : 3;  // steps the loads cover
    static constexpr int begin = KK > kSpread ? kTotal : kTotal * (KK - 1) / kSpread;
    static constexpr int end = KK >= kSpread ? kTotal : kTotal * KK / kSpread;
    // Range of this loader's own issue indices inside [begin, end).
    static constexpr int lo = Loader == 0 ? (begin < kA ? begin : kA) : (begin > kA ? begin - kA : 0);
    static constexpr int hi = Loader == 0 ? (end < kA ? end : kA) : (end > kA ? end - kA : 0);
    static constexpr int count = hi > lo ? hi - lo : 0;
  };

  template <int KK>
  __device__ __forceinline__ static void issue_share(ALoader& la, BLoader& lb,
                                                     __amdgpu_buffer_rsrc_t ra,
                                                     __amdgpu_buffer_rsrc_t rb, char* nxt,
                                                     const TileJob& j, int tid, int k0,
                                                     int Ki) {
    using SA = Share<0, KK>;
    using SB = Share<1, KK>;
    if constexpr (SA::count > 0)
      la.template issue<SA::lo, SA::hi>(ra, nxt, tid, j.m_valid, k0, Ki);
    if constexpr (SB::count > 0)
      lb.template issue<SB::lo, SB::hi>(rb, nxt + kATileBytes, tid, j.n_valid, k0, Ki);
  }

  template <int KK>
  static constexpr int vmem_count() {
    return (AMn ? 0 : Share<0, KK>::count) + (BMn ? 0 : Share<1, KK>::count);
  }

  // One K tile: compute on stage `cur` while the next tile loads into `nxt`.
  //
  // The loads of tile kt+1 go into `nxt` (last read before the previous
  // barrier), spread over the first three 16-wide K steps; each step reads
  // the next step's fragments while its own MFMAs run.  The barrier sits
  // before the last step's MFMAs: by then every wave has issued (and, by the
  // barrier's LDS wait, completed) all its reads of `cur`, and its own loads
  // into `nxt` have landed, so the last step can already read `nxt`'s first
  // fragments.  `cur` and `nxt` are distinct __shared__ objects, which lets
  // the compiler see that reads of one never alias the direct-to-LDS writes
  // into the other (otherwise it waits for those loads before every read).
  __device__ __forceinline__ static void k_tile(f32x16 (&acc)[kFM][kFN], Frags& f0,
                                                Frags& f1, ALoader& la, BLoader& lb,
                                                __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, char* cur,
                                                char* nxt, const TileJob& j, int tid,
                                                const FragOffsets& o, int kt, int kt_total,
                                                int Ki) {
    // The loads are unconditional so that they share a basic block with the
    // MFMAs they interleave with; after the last tile they start at k = K,
    // where every chunk is out of range and fills `nxt` (read by nobody
    // again) with zeros.
    const int k1 = kt + 1 < kt_total ? (kt + 1) * kBK : Ki;
    issue_share<1>(la, lb, ra, rb, nxt, j, tid, k1, Ki);
    step<vmem_count<1>()>(acc, f0, f1, cur, cur + kATileBytes, o, 1);
    issue_share<2>(la, lb, ra, rb, nxt, j, tid, k1, Ki);
    step<vmem_count<2>()>(acc, f1, f0, cur, cur + kATileBytes, o, 2);
    issue_share<3>(la, lb, ra, rb, nxt, j, tid, k1, Ki);
    step<vmem_count<3>()>(acc, f0, f1, cur, cur + kATileBytes, o, 3);
    la.commit(nxt, tid);
    lb.commit(nxt + kATileBytes, tid);
    wait_vmem();
    __syncthreads();
    // After the last tile this reads stale LDS into f0, which is never
    // used; keeping the step unconditional keeps the accumulators out of any
    // control-flow merge (which would cost register copies).
    step<0>(acc, f1, f0, nxt, nxt + kATileBytes, o, 0);
  }

  // Runs the mainloop over K and the epilogue for one tile; s0 and s1 are
  // the two LDS stages (kStageBytes each).
  __device__ __forceinline__ static void run(char* s0, char* s1, const TileJob& j,
                                             int64_t K, const void* C,
                                             int c_dtype, void* D, int d_dtype,
                                             int64_t ldd) {
    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; readfirstlane lets the
    // compiler keep it (and every LDS base derived from it) in SGPRs.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int lrow = lane & 31, lhalf = lane >> 5;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(j.a, j.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(j.b, j.b_bytes);

    f32x16 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int k = 0; k < kFN; ++k) acc[i][k] = f32x16{};

    const int Ki = (int)K;
    const int kt_total = (Ki + kBK - 1) / kBK;
    ALoader la;
    BLoader lb;
    la.init(tid, j.a_pitch);
    lb.init(tid, j.b_pitch);
    if (kt_total > 0) {
      la.issue(ra, s0, tid, j.m_valid, 0, Ki);
      lb.issue(rb, s0 + kATileBytes, tid, j.n_valid, 0, Ki);
      la.commit(s0, tid);
      lb.commit(s0 + kATileBytes, tid);
    }
    wait_vmem();
    __syncthreads();

    const FragOffsets o = frag_offsets(wm, wn, lrow, lhalf);
    Frags f0, f1;
    if (kt_total > 0) read_frags(f0, s0, s0 + kATileBytes, o, 0);

    // Two K tiles per trip so that each tile's stage is a fixed object; an
    // odd last tile is peeled (an exit between the two tiles of a trip makes
    // the register allocator spill the accumulators).
    int kt = 0;
    for (; kt + 1 < kt_total; kt += 2) {
      k_tile(acc, f0, f1, la, lb, ra, rb, s0, s1, j, tid, o, kt, kt_total, Ki);
      k_tile(acc, f0, f1, la, lb, ra, rb, s1, s0, j, tid, o, kt + 1, kt_total, Ki);
    }
    if (kt < kt_total) k_tile(acc, f0, f1, la, lb, ra, rb, s0, s1, j, tid, o, kt, kt_total, Ki);

    epilogue(acc, j, C, c_dtype, D, d_dtype, ldd, lane, wm, wn);
  }

  // Accumulator layout of v_mfma_f32_32x32x*: lane l, register r holds MFMA
  // row 8*(r/4) + 4*(l/32) + r%4 and column l%32; with the operand swap
  // above that is n = 8q + 4*(l/32) + {0..3} (q = r/4) and m = l%32.
  //
  // The element types are dispatched once per tile.  Each 32-row block of
  // the wave's output is 4*kFN chunks of 4 consecutive n per lane; the C
  // chunks of block fm+1 are loaded while block fm is added and stored, and
  // the loads are unconditional (row and column clamped into the tile: a
  // clamped chunk is read but never stored; D's row pitch makes N, hence
  // every tile's valid width, a multiple of 4), so the block's loads go out
  // together and the wave waits for memory once per block rather than once
  // per chunk.
  __device__ __forceinline__ static void epilogue(const f32x16 (&acc)[kFM][kFN],
                                                  const TileJob& j, const void* C,
                                                  int c_dtype, void* D, int d_dtype,
                                                  int64_t ldd, int lane, int wm,
                                                  int wn) {
    const int cd = C ? c_dtype : SG_NONE;
    if (d_dtype == SG_F32) {
      if (cd == SG_F32) return epilogue_t<SG_F32, SG_F32>(acc, j, C, D, ldd, lane, wm, wn);
      if (cd == SG_BF16) return epilogue_t<SG_BF16, SG_F32>(acc, j, C, D, ldd, lane, wm, wn);
      if (cd == SG_F16) return epilogue_t<SG_F16, SG_F32>(acc, j, C, D, ldd, lane, wm, wn);
      return epilogue_t<SG_NONE, SG_F32>(acc, j, C, D, ldd, lane, wm, wn);
    }
    if (d_dtype == SG_BF16) {
      if (cd == SG_F32) return epilogue_t<SG_F32, SG_BF16>(acc, j, C, D, ldd, lane, wm, wn);
      if (cd == SG_BF16) return epilogue_t<SG_BF16, SG_BF16>(acc, j, C, D, ldd, lane, wm, wn);
      if (cd == SG_F16) return epilogue_t<SG_F16, SG_BF16>(acc, j, C, D, ldd, lane, wm, wn);
      return epilogue_t<SG_NONE, SG_BF16>(acc, j, C, D, ldd, lane, wm, wn);
    }
    if (cd == SG_F32) return epilogue_t<SG_F32, SG_F16>(acc, j, C, D, ldd, lane, wm, wn);
    if (cd == SG_BF16) return epilogue_t<SG_BF16, SG_F16>(acc, j, C, D, ldd, lane, wm, wn);
    if (cd == SG_F16) return epilogue_t<SG_F16, SG_F16>(acc, j, C, D, ldd, lane, wm, wn);
    return epilogue_t<SG_NONE, SG_F16>(acc, j, C, D, ldd, lane, wm, wn);
  }

  template <int CD>
  using CChunk = c_chunk_t<CD>;

  template <int CD>
  __device__ __forceinline__ static void load_c_block(CChunk<CD> (&c)[4 * kFN],
                                                      const TileJob& j, const void* C,
                                                      int64_t ldd, int lane, int wm, int wn,
                                                      int fm) {
    if constexpr (CD != SG_NONE) {
      const int ml = min(wm * kWM + fm * 32 + (lane & 31), j.m_valid - 1);
      const int64_t base = (j.d_row0 + ml) * j.ldc + j.n0;
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = min(wn * kWN + fn * 32 + 8 * q + 4 * (lane >> 5), j.n_valid - 4);
          c[4 * fn + q] = load_c_chunk<CD>(C, base + nl);
        }
    }
  }

  template <int CD, int DD>
  __device__ __forceinline__ static void epilogue_t(const f32x16 (&acc)[kFM][kFN],
                                                    const TileJob& j, const void* C, void* D,
                                                    int64_t ldd, int lane, int wm, int wn) {
    CChunk<CD> cb[2][4 * kFN];
    load_c_block<CD>(cb[0], j, C, ldd, lane, wm, wn, 0);
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm) {
      if (fm + 1 < kFM) load_c_block<CD>(cb[(fm + 1) & 1], j, C, ldd, lane, wm, wn, fm + 1);
      const int ml = wm * kWM + fm * 32 + (lane & 31);
      if (ml >= j.m_valid) continue;
      const int64_t row = j.d_row0 + ml;
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * kWN + fn * 32 + 8 * q + 4 * (lane >> 5);
          if (nl >= j.n_valid) continue;
          const int64_t idx = row * ldd + j.n0 + nl;
          const f32x4 v = {acc[fm][fn][4 * q + 0], acc[fm][fn][4 * q + 1],
                           acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
          store_d_chunk<CD, DD>(v, cb[fm & 1][4 * fn + q], D, idx, j.alpha, j.beta);
        }
      }
    }
  }
};

// Workgroup -> output tile of the dense GEMM and the operand panels it
// reads (XCD-aware remap, then the GROUP_M raster).
template <int BM, int BN, bool AMn, bool BMn>
__device__ __forceinline__ TileJob dense_tile_job(const DenseParams& p, int wg) {
  const int total = p.tiles_m * p.tiles_n;
  const int t = xcd_remap(wg, total);
  int tm, tn;
  raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  TileJob j;
  const int64_t es = 2;
  j.m_valid = (int)min<int64_t>(BM, p.M - m0);
  j.n_valid = (int)min<int64_t>(BN, p.N - n0);
  // Each buffer covers exactly the bytes the tile may read: up to the end of
  // its last valid row (K-major) or of row K-1 (MN-major).
  if constexpr (AMn) {  // A stored [K][lda], M contiguous
    j.a = static_cast<const char*>(p.A) + m0 * es;
    j.a_pitch = (uint32_t)(p.lda * es);
    j.a_bytes = p.K > 0 ? (uint32_t)((p.K - 1) * p.lda * es + (p.M - m0) * es) : 0u;
  } else {              // A stored [M][lda], K contiguous
    j.a = static_cast<const char*>(p.A) + m0 * p.lda * es;
    j.a_pitch = (uint32_t)(p.lda * es);
    j.a_bytes = p.K > 0 ? (uint32_t)((j.m_valid - 1) * p.lda * es + p.K * es) : 0u;
  }
  if constexpr (BMn) {  // B stored [K][ldb], N contiguous
    j.b = static_cast<const char*>(p.B) + n0 * es;
    j.b_pitch = (uint32_t)(p.ldb * es);
    j.b_bytes = p.K > 0 ? (uint32_t)((p.K - 1) * p.ldb * es + (p.N - n0) * es) : 0u;
  } else {              // B stored [N][ldb], K contiguous
    j.b = static_cast<const char*>(p.B) + n0 * p.ldb * es;
    j.b_pitch = (uint32_t)(p.ldb * es);
    j.b_bytes = p.K > 0 ? (uint32_t)((j.n_valid - 1) * p.ldb * es + p.K * es) : 0u;
  }
  j.ldc = p.ldc;
  j.alpha = p.alpha;
  j.beta = p.beta;
  j.d_row0 = m0;
  j.n0 = n0;
  return j;
}

// Workgroup -> (group, output tile) of the grouped GEMM (A rows of group g
// are [m_off[g], m_off[g+1]), B of group g is [N][K] at g*N*K).
template <int BM, int BN>
__device__ __forceinline__ TileJob grouped_tile_job(const GroupedParams& p, int wg) {
  const int total = p.tile_start[p.G];
  const int t = xcd_remap(wg, total);
  // Group of tile t: the last g with tile_start[g] <= t (binary search).
  int lo = 0, hi = p.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int64_t Mg = p.m_off[g + 1] - p.m_off[g];
  const int tiles_m = (int)((Mg + BM - 1) / BM);
  int tm, tn;
  raster(t - p.tile_start[g], tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  TileJob j;
  const int64_t es = 2;
  j.m_valid = (int)min<int64_t>(BM, Mg - m0);
  j.n_valid = (int)min<int64_t>(BN, p.N - n0);
  j.a = static_cast<const char*>(p.A) + (p.m_off[g] + m0) * p.K * es;
  j.a_pitch = (uint32_t)(p.K * es);
  j.a_bytes = (uint32_t)(j.m_valid * p.K * es);
  j.b = static_cast<const char*>(p.B) + ((int64_t)g * p.N + n0) * p.K * es;
  j.b_pitch = (uint32_t)(p.K * es);
  j.b_bytes = (uint32_t)(j.n_valid * p.K * es);
  j.d_row0 = p.m_off[g] + m0;
  j.n0 = n0;
  j.ldc = 0;
  j.alpha = 1.0f;
  j.beta = 0.0f;
  return j;
}

template <int BM, int BN, bool IsBF16, bool AMn, bool BMn, int Swz, int Waves>
__global__ void __launch_bounds__(64 * Waves, 1)
    dense_gemm_kernel(const DenseParams p) {
  using Tile = GemmTile<BM, BN, IsBF16, AMn, BMn, Swz, Waves>;
  __shared__ __attribute__((aligned(4096))) char s0[Tile::kStageBytes];
  __shared__ __attribute__((aligned(4096))) char s1[Tile::kStageBytes];

  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = dense_tile_job<BM, BN, AMn, BMn>(p, blockIdx.x);
  Tile::run(s0, s1, j, p.K, p.C, p.c_dtype, p.D, p.d_dtype, p.ldd);
  clock_end(p.clk, cs);
}

template <int BM, int BN, bool IsBF16, int Swz, int Waves>
__global__ void __launch_bounds__(64 * Waves, 1)
    grouped_gemm_kernel(const GroupedParams p) {
  using Tile = GemmTile<BM, BN, IsBF16, false, false, Swz, Waves>;
  __shared__ __attribute__((aligned(4096))) char s0[Tile::kStageBytes];
  __shared__ __attribute__((aligned(4096))) char s1[Tile::kStageBytes];

  const ClockStamp cs = clock_begin(p.clk);
  const TileJob j = grouped_tile_job<BM, BN>(p, blockIdx.x);
  Tile::run(s0, s1, j, p.K, nullptr, SG_NONE, p.D, p.d_dtype, p.N);
  clock_end(p.clk, cs);
}

}  // namespace sg
