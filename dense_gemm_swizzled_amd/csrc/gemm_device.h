// gemm_device.h -- device building blocks of the swizzled GEMM kernels
// (gfx950 / CDNA4): vector types, the LDS swizzle, buffer loads with
// hardware out-of-range zero fill, the operand-tile loaders and the MFMA
// wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_layout.h"

namespace sg {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaveSize = 64;
constexpr int kThreads = 256;  // default workgroup: 4 waves

// Byte offset past every extent the library accepts: a buffer load there
// returns zeros (raw buffer range check), which is how ragged M/N/K edges
// and K tails are filled.
constexpr uint32_t kOutOfRange = 0x80000000u;

// gfx9 buffer descriptor word 3: 32-bit data format, raw (stride 0) access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r,
                                               uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The same with an SGPR byte offset added to the address.  The range check
// may leave the SGPR offset out: off + soff must lie inside the buffer.
__device__ __forceinline__ u32x4 buffer_load16_so(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                  uint32_t soff) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                 r, off, (int)__builtin_amdgcn_readfirstlane(soff), 0));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r,
                                                 uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load2(__amdgpu_buffer_rsrc_t r,
                                                 uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// LDS access in 16-byte units (the swizzle never splits a 16-byte atom).
__device__ __forceinline__ u32x4 lds_read16(const char* lds, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(lds + off);
}
// An 8-byte LDS read kept as its own ds_read_b64: a volatile access is never
// merged with another into a ds_read2 (whose two results sit in adjacent
// registers, which would keep them out of two different operand tuples).
__device__ __forceinline__ u32x2 lds_read8(const char* lds, uint32_t off) {
  typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2;
  return *(lds_u32x2*)(lds + off);
}
__device__ __forceinline__ void lds_write8(char* lds, uint32_t off, u32x2 v) {
  *reinterpret_cast<u32x2*>(lds + off) = v;
}
__device__ __forceinline__ void lds_write16(char* lds, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}

// ---------------------------------------------------------------------------
// Clock trace (measurement only).  When `buf` is non-NULL, workgroup b <
// `slots` records the shader-clock counter (s_memtime) and the constant-rate
// real-time counter (s_memrealtime) when it starts and when its first wave
// has finished, as buf[4b .. 4b+3] = {t_start, t_end, rt_start, rt_end}; the
// ratio of the two deltas, times the real-time counter's rate, is the clock
// the workgroup ran at.  With `buf` NULL the kernels only test the pointer.
// ---------------------------------------------------------------------------
struct ClockTrace {
  uint64_t* buf;
  int64_t slots;
};

struct ClockStamp {
  uint64_t t, rt;
};

__device__ __forceinline__ ClockStamp clock_begin(const ClockTrace& c) {
  ClockStamp s{0, 0};
  if (c.buf) {
    s.t = __builtin_amdgcn_s_memtime();
    s.rt = __builtin_amdgcn_s_memrealtime();
  }
  return s;
}

__device__ __forceinline__ void clock_end(const ClockTrace& c, const ClockStamp& s) {
  if (c.buf && (int64_t)blockIdx.x < c.slots && threadIdx.x == 0) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    uint64_t* o = c.buf + 4 * (int64_t)blockIdx.x;
    o[0] = s.t;
    o[1] = t;
    o[2] = s.rt;
    o[3] = rt;
  }
}

// ---------------------------------------------------------------------------
// Operand tile loaders.  A tile is `Rows` operand rows (M rows of A or N rows
// of B) by 128 bytes of K (64 fp16/bf16 or 128 fp8 elements), stored in LDS
// K-major as Rows x 128 B under lds_offset<128, Swz>.  Global reads are 16
// bytes per lane; consecutive lanes read consecutive 16-byte chunks of one
// row (coalesced); the swizzle permutes only the LDS destination.
// ---------------------------------------------------------------------------

// Direct global -> LDS loader for a K-major operand tile (Rows x 128 B),
// shared by the workgroup's Waves waves.
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes to LDS at M0 + 16*l,
// so one instruction fills 1 KiB of LDS with no VGPR staging and no
// ds_write.  The tile is cut into Rows/8 regions of 1 KiB; region r =
// Waves*i + wave.  Lane l of a region fills physical bytes [1 KiB*r + 16l,
// +16); the swizzle is an involution, so it fetches the logical chunk whose
// swizzled offset that is.  The XOR key of a 256-byte line is (line index
// mod 16) and a region spans 4 lines, so regions Waves*i + wave share the key
// for every i: the lane's K chunk is fixed and its row advances by 8*Waves.
template <int Rows, int Swz, int Waves = 4>
struct DmaLoader {
  static constexpr int kSteps = Rows / (8 * Waves);  // regions per wave
  static_assert(kSteps * 8 * Waves == Rows, "tile rows must fill the waves' regions");
  uint32_t base;    // row0 * pitch + 16 * chunk
  uint32_t chunk16; // 16 * chunk
  int row0;
  uint32_t pitch;

  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_pitch) {
    const uint32_t phys = (uint32_t)wave * 1024u + 16u * (uint32_t)lane;
    const uint32_t logical = swz_bytes<Swz>(phys);
    row0 = (int)(logical >> 7);
    chunk16 = logical & 127u;
    pitch = row_pitch;
    base = (uint32_t)row0 * row_pitch + chunk16;
  }

  // Issues the loads of K bytes [kbyte0, kbyte0 + 128) of every row into the
  // tile at `lds` (generic pointer to the tile's first byte) for this wave's
  // regions I0 <= i < I1.  Rows at or beyond rows_valid and bytes at or
  // beyond kbytes_total read as zero.
  template <int I0 = 0, int I1 = kSteps>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char* lds, int wave,
                                        int rows_valid, uint32_t kbyte0,
                                        uint32_t kbytes_total) const {
    const bool k_ok = kbyte0 + chunk16 < kbytes_total;
#pragma unroll
    for (int i = I0; i < (I1 < kSteps ? I1 : kSteps); ++i) {
      const bool ok = k_ok && row0 + 8 * Waves * i < rows_valid;
      const uint32_t off =
          ok ? base + (uint32_t)(8 * Waves * i) * pitch + kbyte0 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + (Waves * i + wave) * 1024), 16,
          off, 0, 0, 0);
    }
  }
};

// MN-major source [K][rows] (rows contiguous, 16-bit elements): the tile is
// 64 k-rows x Rows.  Thread t owns the 8x8 block (k-chunk kc = t%8, row
// chunk rc = t/8): it reads 8 k-rows of 16 bytes, transposes the 8x8 block
// of 16-bit values in registers, and writes 8 K-major LDS rows.
template <int Rows>
struct MNMajorLoader {
  static constexpr int kActive = Rows / 8 * 8;  // threads that own a block
  u32x4 v[8];

  // row_pitch: bytes per k-row of the source (= total rows * 2);
  // cols_valid: tile rows that exist; k0: first k of the tile; K: total k.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int tid,
                                       uint32_t row_pitch, int cols_valid,
                                       int k0, int K) {
    const int kc = tid & 7, rc = tid >> 3;
    const bool c_ok = tid < kActive && rc * 8 < cols_valid;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + kc * 8 + j;
      const bool ok = c_ok && k < K;
      v[j] = buffer_load16(r, ok ? (uint32_t)k * row_pitch + 16u * rc
                                 : kOutOfRange);
    }
  }

  template <int Swz>
  __device__ __forceinline__ void store(char* lds, int tid) const {
    if (tid >= kActive) return;
    const int kc = tid & 7, rc = tid >> 3;
    // v[j] holds k-row j, columns 0..7 of the block as 4 dwords of 2 values
    // (even column in the low half).  Output row c needs column c of every
    // k-row: dword q of row c = { v[2q] col c, v[2q+1] col c }.
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = __builtin_amdgcn_perm(v[2 * q + 1][c >> 1], v[2 * q][c >> 1], sel);
      lds_write16(lds, lds_offset<128, Swz>(rc * 8 + c, kc), o);
    }
  }
};

// One operand's loader with a common interface: issue() starts the global
// reads of one K tile into an LDS tile, commit() finishes it (a no-op for the
// direct-to-LDS path, the transposed ds_writes for MN-major sources).
// ElemBytes = 2 for fp16/bf16, 1 for fp8.
template <int Rows, bool Mn, int Swz, int ElemBytes, int Waves = 4>
struct OperandLoader;

template <int Rows, int Swz, int ElemBytes, int Waves>
struct OperandLoader<Rows, false, Swz, ElemBytes, Waves> {
  static constexpr int kIssues = DmaLoader<Rows, Swz, Waves>::kSteps;  // loads per thread
  DmaLoader<Rows, Swz, Waves> d;
  __device__ __forceinline__ void init(int tid, uint32_t pitch) {
    d.init(__builtin_amdgcn_readfirstlane(tid >> 6), tid & 63, pitch);
  }
  // Issues this thread's loads I0 <= i < I1 of one K tile.
  template <int I0 = 0, int I1 = kIssues>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char* lds, int tid,
                                        int rows_valid, int k0, int K) {
    d.template issue<I0, I1>(r, lds, __builtin_amdgcn_readfirstlane(tid >> 6), rows_valid,
                             (uint32_t)k0 * ElemBytes, (uint32_t)K * ElemBytes);
  }
  __device__ __forceinline__ void commit(char*, int) const {}
};

// K-major operand tile for the padded layout: the direct-to-LDS path fills
// 1 KiB of consecutive LDS per instruction, which padded rows do not tile,
// so each thread loads 16-byte chunks into registers (consecutive threads
// along a row: coalesced) and writes them to their padded place.  Thread t
// owns chunk t%8 of rows t/8 + (64 Waves / 8) i.
template <int Rows, int ElemBytes, int Waves>
struct OperandLoader<Rows, false, kSwzPad, ElemBytes, Waves> {
  static constexpr int kRowsPerPass = 64 * Waves / 8;
  static constexpr int kIssues = Rows / kRowsPerPass;  // loads per thread
  static_assert(kIssues * kRowsPerPass == Rows, "tile rows must fill the passes");
  u32x4 v[kIssues];
  uint32_t pitch;
  __device__ __forceinline__ void init(int, uint32_t p) { pitch = p; }
  template <int I0 = 0, int I1 = kIssues>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char*, int tid,
                                        int rows_valid, int k0, int K) {
    const int chunk = tid & 7;
    const uint32_t kb = (uint32_t)k0 * ElemBytes + 16u * (uint32_t)chunk;
    const bool k_ok = kb < (uint32_t)K * ElemBytes;
#pragma unroll
    for (int i = I0; i < (I1 < kIssues ? I1 : kIssues); ++i) {
      const int row = (tid >> 3) + kRowsPerPass * i;
      v[i] = buffer_load16(r, k_ok && row < rows_valid ? (uint32_t)row * pitch + kb
                                                        : kOutOfRange);
    }
  }
  __device__ __forceinline__ void commit(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kIssues; ++i)
      lds_write16(lds, lds_offset<128, kSwzPad>((tid >> 3) + kRowsPerPass * i, tid & 7), v[i]);
  }
};

template <int Rows, int Swz, int ElemBytes, int Waves>
struct OperandLoader<Rows, true, Swz, ElemBytes, Waves> {
  static_assert(ElemBytes == 2, "MN-major sources are 16-bit");
  static constexpr int kIssues = 1;  // one batch of register loads
  MNMajorLoader<Rows> m;
  uint32_t pitch;
  __device__ __forceinline__ void init(int, uint32_t p) { pitch = p; }
  template <int I0 = 0, int I1 = kIssues>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char*, int tid,
                                        int rows_valid, int k0, int K) {
    if constexpr (I0 == 0 && I1 > 0) m.load(r, tid, pitch, rows_valid, k0, K);
  }
  __device__ __forceinline__ void commit(char* lds, int tid) const {
    m.template store<Swz>(lds, tid);
  }
};

__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// MFMA wrappers (v_mfma_f32_32x32x16_{bf16,f16}, v_mfma_scale_f32_32x32x64_
// f8f6f4).  Operand lane layout used throughout: lane l supplies row l%32 of
// its operand and the 16-byte K chunk l/32 of the current K step; A and B use
// the same K assignment, so the product is independent of how the hardware
// orders K inside the instruction.
// ---------------------------------------------------------------------------
template <bool IsBF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IsBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row l%16 of its operand and
// the 16-byte K chunk l/16 of the 32-wide K step; lane l receives rows
// 4(l/16) .. 4(l/16)+3 of column l%16 of the 16x16 result.
template <bool IsBF16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (IsBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Epilogue element conversions (round to nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Converts with v_cvt_pk_bf16_f32 (round to nearest even).
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

}  // namespace sg
