// Device-only translation unit for the assembly lint in
// tests/test_asm_lint_cpu.py: instantiates the kernels whose direct-to-LDS
// loads take m0 from a separate, earlier write.
#include "../../dense_gemm_swizzled_amd/csrc/pingpong16.h"

namespace sg {
template __global__ void pingpong16_gemm_kernel<true, 16, false, false, true>(const DenseParams);
template __global__ void pingpong16_gemm_kernel<false, 16, false, true, true>(const DenseParams);
template __global__ void pingpong16_grouped_kernel<true, 16>(const GroupedParams);
template __global__ void pingpong_mx_kernel<16, 0, false>(const MxParams);
template __global__ void pingpong_mx_kernel<16, 0, true>(const MxParams);
template __global__ void pingpong_mx_kernel<16, 2, false>(const MxParams);
template __global__ void pingpong_mx_kernel<16, 2, true>(const MxParams);
template __global__ void pingpong_mx_kernel<16, 4, false>(const MxParams);
template __global__ void pingpong_mx_kernel<16, 4, true>(const MxParams);
}  // namespace sg
