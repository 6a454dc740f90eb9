// launch.h -- host-side launchers of the kernel variants (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernels.h"
#include "mx_kernels.h"

namespace sg {

// Tile shapes the planner chooses between.
enum TileShape { kTile256 = 0, kTile128 = 1, kTile64 = 2 };

// Launches the dense kernel for (tile, dtype, majorness).  Returns the
// launch status.
hipError_t launch_dense(TileShape tile, bool bf16, bool a_mn, bool b_mn,
                        const DenseParams& p, hipStream_t s);
// The layout ablation: bf16, K-major operands, 256x256 tiles on the 32x32x16
// ping-pong kernel with the LDS layout swz (0, 8 or 16 units per line).
hipError_t launch_layout(int swz, const DenseParams& p, hipStream_t s);
// The same on 128x128 tiles of the 4-wave GemmTile kernel, where the padded
// layout (kSwzPad) also fits: layout 16, 8, 0 or kSwzPad.
hipError_t launch_layout128(int layout, const DenseParams& p, hipStream_t s);
hipError_t launch_grouped(TileShape tile, bool bf16, int swz,
                          const GroupedParams& p, int grid, hipStream_t s);
hipError_t launch_mx(TileShape tile, const MxParams& p, hipStream_t s);
hipError_t launch_mxfp4(const MxParams& p, hipStream_t s);  // 256x256 tiles
hipError_t launch_mxfp6(bool e3m2, const MxParams& p, hipStream_t s);  // 256x256 tiles
hipError_t launch_lds_image(const void* X, int64_t rows_total, int64_t K,
                            int elem_bytes, int64_t row0, int64_t k0,
                            int tile_rows, void* out, hipStream_t s);

}  // namespace sg
