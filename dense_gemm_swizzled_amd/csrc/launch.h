// launch.h -- host-side launchers of the kernel variants (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "gemm_kernels.h"
#include "mx_kernels.h"

namespace sg {

// Tile shapes the planner chooses between.
enum TileShape { kTile256 = 0, kTile128 = 1, kTile64 = 2 };

// Name of the kernel instantiation this thread launched last (set by every
// launcher; read through gemm_last_kernel()).
const char*& last_kernel();

// "name<a,b,...>" built once per instantiation.
template <class... Parts>
const char* kernel_label(const char* name, Parts... parts) {
  std::string s = std::string(name) + "<";
  const char* ps[] = {parts...};
  for (size_t i = 0; i < sizeof...(Parts); ++i) s += (i ? std::string(",") : std::string()) + ps[i];
  s += ">";
  char* out = new char[s.size() + 1];  // one per instantiation, kept for the process
  std::copy(s.begin(), s.end(), out);
  out[s.size()] = 0;
  return out;
}

// Launches the dense kernel for (tile, dtype, majorness).  Returns the
// launch status.
hipError_t launch_dense(TileShape tile, bool bf16, bool a_mn, bool b_mn,
                        const DenseParams& p, hipStream_t s);
// The layout ablation: bf16, K-major operands, 256x256 tiles on the 32x32x16
// ping-pong kernel with the LDS layout swz (0, 8 or 16 units per line).
hipError_t launch_layout(int swz, const DenseParams& p, hipStream_t s);
// The input/output ablation on the library's 256x256 kernel (16x16x32
// MFMAs, 16-bit D staged in LDS): operand layout swz (16 or 0) and the
// epilogue's C/D staging swizzled (out_swz) or in logical order.
hipError_t launch_layout_io(int swz, bool out_swz, const DenseParams& p, hipStream_t s);
// The same on 128x128 tiles of the 4-wave GemmTile kernel, where the padded
// layout (kSwzPad) also fits: layout 16, 8, 0 or kSwzPad.
hipError_t launch_layout128(int layout, const DenseParams& p, hipStream_t s);
hipError_t launch_grouped(TileShape tile, bool bf16, int swz,
                          const GroupedParams& p, int grid, hipStream_t s);
hipError_t launch_mx(TileShape tile, const MxParams& p, hipStream_t s);
hipError_t launch_mxfp4(const MxParams& p, hipStream_t s);  // 256x256 tiles
hipError_t launch_mxfp6(bool e3m2, const MxParams& p, hipStream_t s);  // 256x256 tiles
// e8m0 scales [rows][K/32] (K a multiple of 128) into the blocks layout of
// SfMap (mx_kernels.h).
hipError_t launch_sf_blocks(const void* sf, int64_t rows, int64_t K, void* out, hipStream_t s);
// The MFMA clock probe (diag.hip): one wave per SIMD of 256 CUs.
int clock_probe_waves();
hipError_t launch_clock_probe(int64_t iters, void* out, hipStream_t s);
// LDS images of the 256x256 kernels' loaders and the scaled-MFMA probe
// (diag.hip); kind is one of the SG_IMG_* codes.
hipError_t launch_lds_image_pp(int kind, const char* X, uint32_t x_bytes, uint32_t pitch,
                               int valid, uint32_t kbyte0, uint32_t kbytes_total,
                               uint32_t unshifted, uint32_t t, void* out, hipStream_t s);
hipError_t launch_lds_image_cblock(const void* C, int64_t ldc, int64_t row0, int64_t n0,
                                   int m_valid, int n_valid, void* out, hipStream_t s);
hipError_t launch_mfma_scale_probe(int fmt, const void* a, const void* b, const void* sa,
                                   const void* sb, void* out, hipStream_t s);
hipError_t launch_lds_image(const void* X, int64_t rows_total, int64_t K,
                            int elem_bytes, int64_t row0, int64_t k0,
                            int tile_rows, void* out, hipStream_t s);

}  // namespace sg
