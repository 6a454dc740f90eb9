// diag.hip -- measurement and test kernels that sit beside the GEMM path: the
// MFMA clock probe, LDS images of the 256x256 kernels' loaders and a probe of
// the scaled MFMA's operand layout.  Nothing here is on the path of a GEMM
// call.
#include "launch.h"
#include "pingpong16.h"

namespace sg {

namespace {

constexpr int kProbeBlocks = 256;  // one workgroup per CU (see the LDS below)
constexpr int kProbeWaves = 8;     // two waves per SIMD, as the 256x256 GEMM runs

__device__ __forceinline__ f32x4 probe_mfma(u32x4 a, u32x4 b, f32x4 c) {
  return mfma16x16x32<true>(a, b, c);
}

// Every wave issues `iters` rounds of eight independent
// v_mfma_f32_16x16x32_bf16 on random bf16 operands held in registers, so the
// MFMA pipes stay busy, and reads the shader-clock counter (s_memtime) and
// the real-time counter (s_memrealtime) around the loop.  Eight waves of 64
// lanes per workgroup with at most 256 registers each keep the accumulators
// in VGPRs (as in the GEMM), so the loop is the eight MFMAs and a counter;
// the 96 KiB of LDS keep a second workgroup off the CU.  out[4w .. 4w+3] of
// wave w = {shader-clock counter at the loop's start, at its end, real-time
// counter at the start, at the end}; out[4 W + w] (W waves) = bits of the
// wave's accumulator sum (keeps the MFMAs live).
__global__ void __launch_bounds__(64 * kProbeWaves, 1)
    clock_probe_kernel(int iters, uint64_t* out) {
  __shared__ char pad[96 * 1024];
  pad[threadIdx.x] = (char)threadIdx.x;

  // xorshift32 per lane; bf16 values with random sign and mantissa and a
  // biased exponent in [120, 127] (magnitudes in [2^-7, 2)).
  uint32_t x = 0x9E3779B9u * (uint32_t)(blockIdx.x * blockDim.x + threadIdx.x + 1);
  auto rnd = [&]() {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  };
  auto bf16x2 = [&]() {
    const uint32_t r = rnd();
    const uint32_t lo = (r & 0x8000u) | ((120u + (r & 7u)) << 7) | ((r >> 3) & 0x7fu);
    const uint32_t hi = ((r >> 16) & 0x8000u) | ((120u + ((r >> 16) & 7u)) << 7) |
                        ((r >> 19) & 0x7fu);
    return lo | (hi << 16);
  };
  const u32x4 a0{bf16x2(), bf16x2(), bf16x2(), bf16x2()};
  const u32x4 a1{bf16x2(), bf16x2(), bf16x2(), bf16x2()};
  const u32x4 b0{bf16x2(), bf16x2(), bf16x2(), bf16x2()};
  const u32x4 b1{bf16x2(), bf16x2(), bf16x2(), bf16x2()};
  f32x4 c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
  __syncthreads();

  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = probe_mfma(a0, b0, c0);
    c1 = probe_mfma(a1, b0, c1);
    c2 = probe_mfma(a0, b1, c2);
    c3 = probe_mfma(a1, b1, c3);
    c4 = probe_mfma(a0, b0, c4);
    c5 = probe_mfma(a1, b0, c5);
    c6 = probe_mfma(a0, b1, c6);
    c7 = probe_mfma(a1, b1, c7);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();

  const f32x4 sum4 = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float sum = (float)pad[(threadIdx.x + 1) & 255] + sum4[0] + sum4[1] + sum4[2] + sum4[3];
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    uint64_t* o = out + 4 * (int64_t)w;
    o[0] = t0;
    o[1] = t1;
    o[2] = r0;
    o[3] = r1;
    out[4 * kProbeBlocks * kProbeWaves + w] = (uint64_t)__builtin_bit_cast(uint32_t, sum);
  }
}

}  // namespace

int clock_probe_waves() { return kProbeBlocks * kProbeWaves; }

hipError_t launch_clock_probe(int64_t iters, void* out, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(kProbeBlocks), dim3(64 * kProbeWaves), 0, s,
                     (int)iters, static_cast<uint64_t*>(out));
  return hipGetLastError();
}

}  // namespace sg

// ---------------------------------------------------------------------------
// LDS images of the 256x256 kernels' loaders.  Each kernel below runs the
// loader code of the GEMM kernels once, as group 0 of a tile (waves 0-3)
// issues it, waits for the loads, and copies the LDS it filled out byte for
// byte.  The images show where each loaded byte lands, which must be where
// the fragment reads look for it.
// ---------------------------------------------------------------------------

namespace sg {

namespace {

constexpr int kImgThreads = 256;  // group 0's four waves

__device__ __forceinline__ void copy_out(const char* smem, int bytes, char* out) {
  for (int i = threadIdx.x; i < bytes / 16; i += kImgThreads)
    reinterpret_cast<u32x4*>(out)[i] = reinterpret_cast<const u32x4*>(smem)[i];
}

// One K-major half tile (128 rows x 128 bytes) through HalfLoader (K checked
// per load) or KExactHalfLoader (row offsets fixed, K position in the SGPR
// offset), as the 16-bit ping-pong loads rows [128g, 128g + 128) of a tile.
template <bool KExact>
__global__ void __launch_bounds__(kImgThreads, 1)
    img_half_kernel(const char* X, uint32_t x_bytes, uint32_t pitch, int rows_valid,
                    uint32_t kbyte0, uint32_t kbytes_total, char* out) {
  __shared__ __attribute__((aligned(4096))) char smem[16384];
  const int lane = threadIdx.x & 63, w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 rsrc = rsrc_words(X, x_bytes);
  const uint32_t half = lds_addr(smem);
  HalfLoader<kSwzDefault> h;
  h.init(w4, lane, pitch);
  if constexpr (KExact) {
    KExactHalfLoader<kSwzDefault> x;
    x.init(h, rows_valid);
    x.issue<0>(rsrc, half, w4, kbyte0);
    x.issue<1>(rsrc, half, w4, kbyte0);
    x.issue<2>(rsrc, half, w4, kbyte0);
    x.issue<3>(rsrc, half, w4, kbyte0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) h.issue(rsrc, half, w4, i, rows_valid, kbyte0, kbytes_total);
  }
  wait_vmem();
  __syncthreads();
  copy_out(smem, 16384, out);
}

// One MN-major half tile of the 16-bit ping-pong: 64 k rows x 128 columns
// (256 bytes), K tile t of the operand, through PingPong16Tile::init_bmn and
// the K-exact loads (64 rows a tile in the SGPR offset).
__global__ void __launch_bounds__(kImgThreads, 1)
    img_mn256_kernel(const char* X, uint32_t x_bytes, uint32_t pitch, int cols_valid,
                     uint32_t t, char* out) {
  __shared__ __attribute__((aligned(4096))) char smem[16384];
  using Tile = PingPong16Tile<true, kSwzDefault, false, true>;
  const int lane = threadIdx.x & 63, w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 rsrc = rsrc_words(X, x_bytes);
  const uint32_t half = lds_addr(smem);
  KExactHalfLoader<kSwzDefault> x;
  Tile::init_bmn(x, 0, w4, lane, pitch, cols_valid);
  const uint32_t kstep = 64u * pitch;
  x.issue<0>(rsrc, half, w4, t * kstep);
  x.issue<1>(rsrc, half, w4, t * kstep);
  x.issue<2>(rsrc, half, w4, t * kstep);
  x.issue<3>(rsrc, half, w4, t * kstep);
  wait_vmem();
  __syncthreads();
  copy_out(smem, 16384, out);
}

// One MXFP6 half tile (128 rows x 96 bytes of a K tile) through the MX
// ping-pong's Fp6Loader, rows [0, 128) of a 256-row tile.
__global__ void __launch_bounds__(kImgThreads, 1)
    img_fp6_kernel(const char* X, uint32_t x_bytes, uint32_t pitch, int rows_valid,
                   uint32_t unshifted, uint32_t t, char* out) {
  __shared__ __attribute__((aligned(4096))) char smem[16384];
  using Tile = PingPongMxTile<kSwzDefault, 2, false>;
  const int lane = threadIdx.x & 63, w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 rsrc = rsrc_words(X, x_bytes);
  const uint32_t half = lds_addr(smem);
  typename Tile::Fp6Loader x;
  x.init(w4, lane, pitch, rows_valid, unshifted);
  const uint32_t kbyte0 = t * 96u;
  x.template issue<0>(rsrc, half, w4, kbyte0);
  x.template issue<1>(rsrc, half, w4, kbyte0);
  x.template issue<2>(rsrc, half, w4, kbyte0);
  x.template issue<3>(rsrc, half, w4, kbyte0);
  wait_vmem();
  __syncthreads();
  copy_out(smem, 16384, out);
}

// The C blocks of group 0's four waves of a 256x256 tile (rows 0..127 of
// the tile, columns 64 w4 .. +63) through the 16-bit ping-pong's CBlock
// quarters, quarter Q into bytes [16384 Q, +16384) of the image.
__global__ void __launch_bounds__(kImgThreads, 1)
    img_cblock_kernel(const void* C, int64_t ldc, int64_t d_row0, int64_t n0, int m_valid,
                      int n_valid, char* out) {
  __shared__ __attribute__((aligned(4096))) char smem[65536];
  using Tile = PingPong16Tile<true, kSwzDefault>;
  const int lane = threadIdx.x & 63, w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  TileJob j{};
  j.d_row0 = d_row0;
  j.n0 = n0;
  j.ldc = ldc;
  j.m_valid = m_valid;
  j.n_valid = n_valid;
  typename Tile::CBlock cb;
  cb.init(j, C, 0, w4, lane);
  const uint32_t s0 = lds_addr(smem);
#pragma unroll
  for (int Q = 0; Q < 4; ++Q) {
    const KExactHalfLoader<kSwzDefault> x = cb.quarter(Q);
    const uint32_t slot = s0 + 16384u * (uint32_t)Q;
    x.issue<0>(cb.rsrc, slot, w4, 0u);
    x.issue<1>(cb.rsrc, slot, w4, 0u);
    x.issue<2>(cb.rsrc, slot, w4, 0u);
    x.issue<3>(cb.rsrc, slot, w4, 0u);
  }
  wait_vmem();
  __syncthreads();
  copy_out(smem, 65536, out);
}

// One v_mfma_scale_f32_32x32x64_f8f6f4 by one wave: lane l's 32-byte
// operands are a[l], b[l] (srcA, srcB), its scale bytes sa[l], sb[l] (op_sel
// 0: byte 0 of the scale register); out[16 l + r] = accumulator register r
// of lane l, starting from zero.
template <int Fmt>
__global__ void __launch_bounds__(64, 1)
    mfma_scale_probe_kernel(const i32x8* a, const i32x8* b, const uint8_t* sa,
                            const uint8_t* sb, float* out) {
  const int l = threadIdx.x;
  const f32x16 d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      a[l], b[l], f32x16{}, Fmt, Fmt, 0, (int)sa[l], 0, (int)sb[l]);
#pragma unroll
  for (int r = 0; r < 16; ++r) out[16 * l + r] = d[r];
}

}  // namespace

hipError_t launch_lds_image_pp(int kind, const char* X, uint32_t x_bytes, uint32_t pitch,
                               int valid, uint32_t kbyte0, uint32_t kbytes_total,
                               uint32_t unshifted, uint32_t t, void* out, hipStream_t s) {
  char* o = static_cast<char*>(out);
  switch (kind) {
    case SG_IMG_HALF:
      hipLaunchKernelGGL((img_half_kernel<false>), dim3(1), dim3(kImgThreads), 0, s, X,
                         x_bytes, pitch, valid, kbyte0, kbytes_total, o);
      break;
    case SG_IMG_HALF_KEXACT:
      hipLaunchKernelGGL((img_half_kernel<true>), dim3(1), dim3(kImgThreads), 0, s, X,
                         x_bytes, pitch, valid, kbyte0, kbytes_total, o);
      break;
    case SG_IMG_MN256:
      hipLaunchKernelGGL(img_mn256_kernel, dim3(1), dim3(kImgThreads), 0, s, X, x_bytes,
                         pitch, valid, t, o);
      break;
    case SG_IMG_FP6:
      hipLaunchKernelGGL(img_fp6_kernel, dim3(1), dim3(kImgThreads), 0, s, X, x_bytes, pitch,
                         valid, unshifted, t, o);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lds_image_cblock(const void* C, int64_t ldc, int64_t row0, int64_t n0,
                                   int m_valid, int n_valid, void* out, hipStream_t s) {
  hipLaunchKernelGGL(img_cblock_kernel, dim3(1), dim3(kImgThreads), 0, s, C, ldc, row0, n0,
                     m_valid, n_valid, static_cast<char*>(out));
  return hipGetLastError();
}

hipError_t launch_mfma_scale_probe(int fmt, const void* a, const void* b, const void* sa,
                                   const void* sb, void* out, hipStream_t s) {
  const i32x8* pa = static_cast<const i32x8*>(a);
  const i32x8* pb = static_cast<const i32x8*>(b);
  const uint8_t* psa = static_cast<const uint8_t*>(sa);
  const uint8_t* psb = static_cast<const uint8_t*>(sb);
  float* po = static_cast<float*>(out);
  switch (fmt) {
    case 0:
      hipLaunchKernelGGL(mfma_scale_probe_kernel<0>, dim3(1), dim3(64), 0, s, pa, pb, psa, psb, po);
      break;
    case 2:
      hipLaunchKernelGGL(mfma_scale_probe_kernel<2>, dim3(1), dim3(64), 0, s, pa, pb, psa, psb, po);
      break;
    case 3:
      hipLaunchKernelGGL(mfma_scale_probe_kernel<3>, dim3(1), dim3(64), 0, s, pa, pb, psa, psb, po);
      break;
    case 4:
      hipLaunchKernelGGL(mfma_scale_probe_kernel<4>, dim3(1), dim3(64), 0, s, pa, pb, psa, psb, po);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sg
