// launch_dense.hip -- instantiations and launchers of the 16-bit dense and
// grouped kernels.
#include "launch.h"
#include "pingpong.h"
#include "pingpong16.h"
#include "deep64.h"

namespace sg {

namespace {

// 256x256 tiles with K-major operands run with 8 waves (two per SIMD);
// 128x128 tiles, and tiles with MN-major operands (whose register
// transposes need the registers of a one-wave-per-SIMD layout), with 4.
template <int BM, bool AMn, bool BMn>
constexpr int waves_for() { return BM == 256 && !AMn && !BMn ? 8 : 4; }

constexpr const char* dt_name(bool bf) { return bf ? "bf16" : "f16"; }
constexpr const char* mj_name(bool mn) { return mn ? "mn" : "k"; }
constexpr const char* swz_name(int swz) {
  return swz == 16 ? "swz16" : swz == 8 ? "swz8" : swz == 0 ? "swz0" : "pad16";
}

template <int BM, int BN, bool BF, bool AMn, bool BMn, int Swz>
hipError_t go_dense(const DenseParams& p, hipStream_t s) {
  static const char* const name =
      kernel_label("dense_gemm_kernel", BM == 256 ? "256" : BM == 128 ? "128" : "64",
                   dt_name(BF), mj_name(AMn), mj_name(BMn), swz_name(Swz));
  last_kernel() = name;
  const int grid = p.tiles_m * p.tiles_n;
  constexpr int W = waves_for<BM, AMn, BMn>();
  hipLaunchKernelGGL((dense_gemm_kernel<BM, BN, BF, AMn, BMn, Swz, W>), dim3(grid),
                     dim3(64 * W), 0, s, p);
  return hipGetLastError();
}

// 256x256 tiles with both operands K-major run the ping-pong mainloop with
// 16x16x32 MFMAs.
template <bool BF, int Swz, bool AMn = false, bool BMn = false, bool OutSwz = true>
hipError_t go_pingpong(const DenseParams& p, hipStream_t s) {
  static const char* const name =
      OutSwz ? kernel_label("pingpong16_gemm_kernel", dt_name(BF), mj_name(AMn), mj_name(BMn),
                            swz_name(Swz))
             : kernel_label("pingpong16_gemm_kernel", dt_name(BF), mj_name(AMn), mj_name(BMn),
                            swz_name(Swz), "out_swz0");
  last_kernel() = name;
  hipLaunchKernelGGL((pingpong16_gemm_kernel<BF, Swz, AMn, BMn, OutSwz>),
                     dim3(p.tiles_m * p.tiles_n), dim3(512), 0, s, p);
  return hipGetLastError();
}

// The layout ablation runs the ping-pong mainloop with 32x32x16 MFMAs, the
// kernel its measurements were taken with.
template <int Swz>
hipError_t go_pingpong32(const DenseParams& p, hipStream_t s) {
  static const char* const name = kernel_label("pingpong_gemm_kernel", "bf16", swz_name(Swz));
  last_kernel() = name;
  hipLaunchKernelGGL((pingpong_gemm_kernel<true, Swz>), dim3(p.tiles_m * p.tiles_n),
                     dim3(512), 0, s, p);
  return hipGetLastError();
}

// 64x64 tiles run the eight-stage ring, 128x128 tiles with K-major operands
// the five-stage one.
template <int BM, bool BF, bool AMn, bool BMn>
hipError_t go_deep(const DenseParams& p, hipStream_t s) {
  static const char* const name = kernel_label("deep_gemm_kernel", BM == 128 ? "128" : "64",
                                               dt_name(BF), mj_name(AMn), mj_name(BMn));
  last_kernel() = name;
  hipLaunchKernelGGL((deep_gemm_kernel<BM, BF, AMn, BMn>), dim3(p.tiles_m * p.tiles_n),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; a race only
// repeats the query).
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cache[dev] = cus;
  }
  return cache[dev];
}

template <int BM, int BN, bool BF, int Swz>
hipError_t dense_by_major(bool a_mn, bool b_mn, const DenseParams& p, hipStream_t s) {
  if (BM == 64) {
    if (a_mn) return b_mn ? go_deep<64, BF, true, true>(p, s) : go_deep<64, BF, true, false>(p, s);
    return b_mn ? go_deep<64, BF, false, true>(p, s) : go_deep<64, BF, false, false>(p, s);
  }
  if (!a_mn && !b_mn) {
    if (BM == 256) return go_pingpong<BF, Swz>(p, s);
    // 128x128: the five-stage ring (160 KiB, one workgroup per CU) while the
    // tiles fit in one round of the CUs; beyond that the two-stage kernel
    // (64 KiB, two workgroups per CU) keeps more of them in flight.
    if ((int64_t)p.tiles_m * p.tiles_n <= device_cus()) return go_deep<128, BF, false, false>(p, s);
    return go_dense<BM, BN, BF, false, false, Swz>(p, s);
  }
  // MN-major operands on 256x256 tiles take the ping-pong when K is a
  // multiple of 64 with at least two K tiles (its loader and ring start
  // assume both).
  if (BM == 256 && p.K % 64 == 0 && p.K >= 128) {
    if (!a_mn && b_mn) return go_pingpong<BF, Swz, false, true>(p, s);
    if (a_mn && !b_mn) return go_pingpong<BF, Swz, true, false>(p, s);
    if (a_mn && b_mn) return go_pingpong<BF, Swz, true, true>(p, s);
  }
  // 128x128 tiles with an MN-major operand: the five-stage ring while the
  // tiles fit in one round of the CUs.
  if (BM == 128 && (int64_t)p.tiles_m * p.tiles_n <= device_cus()) {
    if (!a_mn && b_mn) return go_deep<128, BF, false, true>(p, s);
    if (a_mn && !b_mn) return go_deep<128, BF, true, false>(p, s);
    if (a_mn && b_mn) return go_deep<128, BF, true, true>(p, s);
  }
  if (!a_mn && b_mn) return go_dense<BM, BN, BF, false, true, Swz>(p, s);
  if (a_mn && !b_mn) return go_dense<BM, BN, BF, true, false, Swz>(p, s);
  return go_dense<BM, BN, BF, true, true, Swz>(p, s);
}

template <int BM, int BN, int Swz>
hipError_t dense_by_dtype(bool bf16, bool a_mn, bool b_mn, const DenseParams& p,
                          hipStream_t s) {
  return bf16 ? dense_by_major<BM, BN, true, Swz>(a_mn, b_mn, p, s)
              : dense_by_major<BM, BN, false, Swz>(a_mn, b_mn, p, s);
}

}  // namespace

hipError_t launch_dense(TileShape tile, bool bf16, bool a_mn, bool b_mn,
                        const DenseParams& p, hipStream_t s) {
  if (tile == kTile256) return dense_by_dtype<256, 256, 16>(bf16, a_mn, b_mn, p, s);
  if (tile == kTile128) return dense_by_dtype<128, 128, 16>(bf16, a_mn, b_mn, p, s);
  return dense_by_dtype<64, 64, 16>(bf16, a_mn, b_mn, p, s);
}

hipError_t launch_layout(int swz, const DenseParams& p, hipStream_t s) {
  if (swz == 16) return go_pingpong32<16>(p, s);
  if (swz == 8) return go_pingpong32<8>(p, s);
  if (swz == 0) return go_pingpong32<0>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_layout_io(int swz, bool out_swz, const DenseParams& p, hipStream_t s) {
  if (swz == 16)
    return out_swz ? go_pingpong<true, 16, false, false, true>(p, s)
                   : go_pingpong<true, 16, false, false, false>(p, s);
  if (swz == 0)
    return out_swz ? go_pingpong<true, 0, false, false, true>(p, s)
                   : go_pingpong<true, 0, false, false, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_layout128(int layout, const DenseParams& p, hipStream_t s) {
  if (layout == 16) return go_dense<128, 128, true, false, false, 16>(p, s);
  if (layout == 8) return go_dense<128, 128, true, false, false, 8>(p, s);
  if (layout == 0) return go_dense<128, 128, true, false, false, 0>(p, s);
  if (layout == kSwzPad) return go_dense<128, 128, true, false, false, kSwzPad>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_grouped(TileShape tile, bool bf16, int swz, const GroupedParams& p,
                          int grid, hipStream_t s) {
  if (swz != 16) return hipErrorInvalidValue;
  static const char* const names[2][2] = {
      {kernel_label("pingpong16_grouped_kernel", "f16"),
       kernel_label("pingpong16_grouped_kernel", "bf16")},
      {kernel_label("grouped_gemm_kernel", "128", "f16"),
       kernel_label("grouped_gemm_kernel", "128", "bf16")}};
  last_kernel() = names[tile == kTile256 ? 0 : 1][bf16 ? 1 : 0];
  if (tile == kTile256) {
    if (bf16)
      hipLaunchKernelGGL((pingpong16_grouped_kernel<true, 16>), dim3(grid), dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL((pingpong16_grouped_kernel<false, 16>), dim3(grid), dim3(512), 0, s, p);
  } else {
    if (bf16)
      hipLaunchKernelGGL((grouped_gemm_kernel<128, 128, true, 16, 4>), dim3(grid),
                         dim3(64 * 4), 0, s, p);
    else
      hipLaunchKernelGGL((grouped_gemm_kernel<128, 128, false, 16, 4>), dim3(grid),
                         dim3(64 * 4), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sg
