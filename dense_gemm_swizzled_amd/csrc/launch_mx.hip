// launch_mx.hip -- MXFP8 / MXFP6 / MXFP4 kernel launchers and the LDS-image debug kernel.
#include "launch.h"
#include "pingpong.h"

namespace sg {

namespace {

// The 256x256 ping-pong for operand format Fmt, with the scale layout p
// names; `labels` = {rows, blocks}.
template <int Fmt>
hipError_t launch_pingpong_mx(const MxParams& p, hipStream_t s, const char* const (&labels)[2]) {
  const bool blocks = p.sf_layout == SG_SF_BLOCKS;
  last_kernel() = labels[blocks ? 1 : 0];
  const dim3 grid(p.tiles_m * p.tiles_n);
  if (blocks)
    hipLaunchKernelGGL((pingpong_mx_kernel<kSwzDefault, Fmt, true>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((pingpong_mx_kernel<kSwzDefault, Fmt, false>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx(TileShape tile, const MxParams& p, hipStream_t s) {
  static const char* const labels[2] = {kernel_label("pingpong_mx_kernel", "e4m3", "rows"),
                                        kernel_label("pingpong_mx_kernel", "e4m3", "blocks")};
  static const char* const name128 = kernel_label("mx_gemm_kernel", "128", "e4m3");
  if (tile == kTile256) return launch_pingpong_mx<0>(p, s, labels);
  last_kernel() = name128;
  hipLaunchKernelGGL((mx_gemm_kernel<128, 128, kSwzDefault>), dim3(p.tiles_m * p.tiles_n),
                     dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mxfp4(const MxParams& p, hipStream_t s) {
  static const char* const labels[2] = {kernel_label("pingpong_mx_kernel", "e2m1", "rows"),
                                        kernel_label("pingpong_mx_kernel", "e2m1", "blocks")};
  return launch_pingpong_mx<4>(p, s, labels);
}

hipError_t launch_mxfp6(bool e3m2, const MxParams& p, hipStream_t s) {
  static const char* const e2m3[2] = {kernel_label("pingpong_mx_kernel", "e2m3", "rows"),
                                      kernel_label("pingpong_mx_kernel", "e2m3", "blocks")};
  static const char* const e3m2_[2] = {kernel_label("pingpong_mx_kernel", "e3m2", "rows"),
                                       kernel_label("pingpong_mx_kernel", "e3m2", "blocks")};
  return e3m2 ? launch_pingpong_mx<3>(p, s, e3m2_) : launch_pingpong_mx<2>(p, s, e2m3);
}

// One row's 16 scale bytes of a group, blocks 0..15 in order, to the block
// layout's order: the even blocks, then the odd ones (block b at byte
// 8 (b mod 2) + b / 2).  v_perm's selector bytes 0-3 pick the bytes of its
// second operand, 4-7 those of its first.
__device__ __forceinline__ u32x4 even_then_odd(u32x4 v) {
  return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x06040200u),
               __builtin_amdgcn_perm(v[3], v[2], 0x06040200u),
               __builtin_amdgcn_perm(v[1], v[0], 0x07050301u),
               __builtin_amdgcn_perm(v[3], v[2], 0x07050301u)};
}

// The scale bytes of 64 rows and one group of 16 K blocks go to one KiB of
// `out`.  A workgroup of 1024 threads takes rows [64 i, 64 i + 64) and up to
// 16 groups (blockIdx.y), one 16-byte unit per thread: it reads the units
// row by row (contiguous in the rows layout), reorders each (even_then_odd),
// transposes them through LDS (groups 1040 bytes apart, so that the 16
// units of one row fall in different banks) and writes them a group at a
// time (one contiguous KiB each).  Rows past `rows` and blocks past K/32 are
// written as zero.
__global__ void __launch_bounds__(1024) sf_blocks_kernel(const uint32_t* sf, int64_t rows,
                                                         int64_t pitch_dw, int64_t groups,
                                                         u32x4* out) {
  constexpr int kLdsRow = 1040;
  __shared__ __attribute__((aligned(16))) char lds[16 * kLdsRow];
  const int64_t rb = blockIdx.x, g0 = 16 * (int64_t)blockIdx.y;
  const int ng = (int)min<int64_t>(16, groups - g0);
  const int u = threadIdx.x;
  if (u < 64 * ng) {
    const int row = u / ng, g = u - row * ng;
    const int64_t r = rb * 64 + row;
    const int64_t n = pitch_dw - 4 * (g0 + g);  // dwords of the row from the unit's first
    u32x4 v{0u, 0u, 0u, 0u};
    if (r < rows) {
      const uint32_t* src = sf + r * pitch_dw + 4 * (g0 + g);
      if (n >= 4) {
        __builtin_memcpy(&v, src, 16);
      } else {
#pragma unroll
        for (int d = 0; d < 3; ++d)
          if (d < n) v[d] = src[d];
      }
    }
    *reinterpret_cast<u32x4*>(lds + g * kLdsRow + row * 16) = even_then_odd(v);
  }
  __syncthreads();
  if (u < 64 * ng) {
    const int g = u >> 6, row = u & 63;
    out[(rb * groups + g0 + g) * 64 + row] =
        *reinterpret_cast<const u32x4*>(lds + g * kLdsRow + row * 16);
  }
}

hipError_t launch_sf_blocks(const void* sf, int64_t rows, int64_t K, void* out, hipStream_t s) {
  const int64_t groups = (K / 32 + 15) / 16;
  hipLaunchKernelGGL(sf_blocks_kernel,
                     dim3((unsigned)((rows + 63) / 64), (unsigned)((groups + 15) / 16)),
                     dim3(1024), 0, s, static_cast<const uint32_t*>(sf), rows, K / 128, groups,
                     static_cast<u32x4*>(out));
  return hipGetLastError();
}

// Runs the K-major (direct-to-LDS) tile loader once (rows [row0, row0 + Rows), bytes
// [k0*eb, k0*eb + 128) of each row) into LDS under the kernels' swizzle and
// copies the LDS stage out linearly.
template <int Rows>
__global__ void __launch_bounds__(kThreads, 1)
    lds_image_kernel(const char* X, uint32_t x_bytes, uint32_t pitch, int rows_valid,
                     uint32_t kbyte0, uint32_t kbytes_total, char* out) {
  __shared__ __attribute__((aligned(4096))) char smem[Rows * 128];
  const int tid = threadIdx.x;
  DmaLoader<Rows, kSwzDefault> ld;
  ld.init(tid >> 6, tid & 63, pitch);
  ld.issue(make_rsrc(X, x_bytes), smem, tid >> 6, rows_valid, kbyte0, kbytes_total);
  wait_vmem();
  __syncthreads();
  for (int i = tid; i < Rows * 128 / 16; i += kThreads)
    reinterpret_cast<u32x4*>(out)[i] = reinterpret_cast<const u32x4*>(smem)[i];
}

hipError_t launch_lds_image(const void* X, int64_t rows_total, int64_t K, int eb,
                            int64_t row0, int64_t k0, int tile_rows, void* out,
                            hipStream_t s) {
  const char* base = static_cast<const char*>(X) + row0 * K * eb;
  const int64_t rv = rows_total - row0;
  const int rows_valid = (int)(rv < tile_rows ? (rv > 0 ? rv : 0) : tile_rows);
  const uint32_t pitch = (uint32_t)(K * eb);
  const uint32_t bytes = (uint32_t)((int64_t)rows_valid * K * eb);
  if (tile_rows == 256)
    hipLaunchKernelGGL((lds_image_kernel<256>), dim3(1), dim3(kThreads), 0, s, base,
                       bytes, pitch, rows_valid, (uint32_t)(k0 * eb), pitch,
                       static_cast<char*>(out));
  else
    hipLaunchKernelGGL((lds_image_kernel<128>), dim3(1), dim3(kThreads), 0, s, base,
                       bytes, pitch, rows_valid, (uint32_t)(k0 * eb), pitch,
                       static_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace sg
