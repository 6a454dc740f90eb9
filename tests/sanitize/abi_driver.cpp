// abi_driver.cpp -- drives every validation path of the C ABI
// (include/swizzled_gemm.h) on the host, for an AddressSanitizer +
// UndefinedBehaviorSanitizer build of the library's host code.  Every call
// below is rejected (or is a no-op) before the library touches the GPU, so
// the run needs none; host arrays are exactly sized heap buffers, so a read
// past m_offsets or an output map shows up as a sanitizer report.  Exit
// status 0 = every return code as documented and no report.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/swizzled_gemm.h"

static int fails = 0;
#define EXPECT_RC(call, want)                                                          \
  do {                                                                                 \
    const int rc_ = (call);                                                            \
    if (rc_ != (want)) {                                                               \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__,      \
                   __LINE__, #call, rc_, (want), gemm_last_error());                   \
      ++fails;                                                                         \
    }                                                                                  \
  } while (0)

int main() {
  // A 16-byte-aligned fake device address: never dereferenced, since every
  // call here fails validation or is empty.
  void* const P = reinterpret_cast<void*>(uintptr_t{0x10000});
  char* const Pc = static_cast<char*>(P);

  // gemm_run / gemm_strided_run
  EXPECT_RC(gemm_run(-1, 8, 8, P, 0, P, 0, SG_BF16, nullptr, 0, P, SG_F32, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_run(8, 8, 8, nullptr, 0, P, 0, SG_BF16, nullptr, 0, P, SG_F32, nullptr), SG_ERR_NULL);
  EXPECT_RC(gemm_run(8, 8, 8, Pc + 8, 0, P, 0, SG_BF16, nullptr, 0, P, SG_F32, nullptr), SG_ERR_ALIGN);
  EXPECT_RC(gemm_run(8, 8, 12, P, 0, P, 0, SG_BF16, nullptr, 0, P, SG_F32, nullptr), SG_ERR_ALIGN);
  EXPECT_RC(gemm_run(8, 8, 8, P, 3, P, 0, SG_BF16, nullptr, 0, P, SG_F32, nullptr), SG_ERR_MAJOR);
  EXPECT_RC(gemm_run(8, 8, 8, P, 0, P, 0, SG_E4M3, nullptr, 0, P, SG_F32, nullptr), SG_ERR_DTYPE);
  EXPECT_RC(gemm_run(0, 8, 8, nullptr, 0, nullptr, 0, SG_BF16, nullptr, 0, nullptr, SG_F32, nullptr), SG_OK);
  EXPECT_RC(gemm_strided_run(300, 264, 100, 1.f, P, 104, 0, P, 104, 0, SG_BF16, 1.f, nullptr, 264, 0,
                             P, 264, SG_F32, nullptr), SG_ERR_SHAPE);   // K % 8 with K-major
  EXPECT_RC(gemm_strided_run(300, 262, 136, 1.f, P, 136, 0, P, 136, 0, SG_BF16, 1.f, nullptr, 264, 0,
                             P, 264, SG_F32, nullptr), SG_ERR_SHAPE);   // N % 4
  EXPECT_RC(gemm_strided_run(300, 264, 136, 1.f, P, 128, 0, P, 136, 0, SG_BF16, 1.f, nullptr, 264, 0,
                             P, 264, SG_F32, nullptr), SG_ERR_SHAPE);   // lda < K
  EXPECT_RC(gemm_layout_run(4, 256, 256, 64, P, P, nullptr, 0, P, SG_F32, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_layout128_run(5, 256, 256, 64, P, P, nullptr, 0, P, SG_F32, nullptr), SG_ERR_SHAPE);

  // grouped_gemm_run: the offsets are read on the host, G + 1 of them.
  for (int G : {1, 2, 128, 255, 256}) {
    std::vector<int64_t> offs(G + 1, 0);
    EXPECT_RC(grouped_gemm_run(G, offs.data(), 256, 64, P, 0, P, 0, SG_BF16, P, SG_BF16, nullptr),
              SG_OK);  // every group empty: nothing to launch
    offs[G] = -1;
    EXPECT_RC(grouped_gemm_run(G, offs.data(), 256, 64, P, 0, P, 0, SG_BF16, P, SG_BF16, nullptr),
              SG_ERR_GROUPS);
  }
  {
    std::vector<int64_t> offs(258, 0);
    EXPECT_RC(grouped_gemm_run(257, offs.data(), 256, 64, P, 0, P, 0, SG_BF16, P, SG_BF16, nullptr),
              SG_ERR_GROUPS);
    EXPECT_RC(grouped_gemm_run(2, nullptr, 256, 64, P, 0, P, 0, SG_BF16, P, SG_BF16, nullptr),
              SG_ERR_NULL);
  }

  // block-scaled
  EXPECT_RC(mx_gemm_run(256, 256, 96, P, P, P, P, P, SG_BF16, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(mx_gemm_run(256, 256, 256, P, Pc + 2, P, P, P, SG_BF16, nullptr), SG_ERR_ALIGN);
  EXPECT_RC(mxfp4_gemm_run(256, 256, 128, P, P, P, P, P, SG_BF16, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(mxfp6_gemm_run(SG_E4M3, 256, 256, 128, P, P, P, P, P, SG_BF16, nullptr), SG_ERR_DTYPE);
  EXPECT_RC(mxfp6_gemm_run(SG_E2M3, 256, 256, 64, P, P, P, P, P, SG_BF16, nullptr), SG_ERR_SHAPE);

  // host-side layout maps into exactly sized buffers
  for (int rb : {64, 128, 256}) {
    std::vector<int32_t> m(256 * (rb / 16));
    EXPECT_RC(gemm_lds_layout(256, rb, m.data()), SG_OK);
  }
  {
    std::vector<int32_t> m(128 * 12);
    for (int u : {0, 11, 31, 32}) EXPECT_RC(gemm_lds_layout_mxfp6(128, u, m.data()), SG_OK);
    std::vector<int32_t> c(4 * 128 * 8);
    EXPECT_RC(gemm_lds_layout_cblock(c.data()), SG_OK);
    EXPECT_RC(gemm_lds_layout(12, 128, m.data()), SG_ERR_SHAPE);
    EXPECT_RC(gemm_lds_layout_cblock(nullptr), SG_ERR_NULL);
  }

  // measurement and test exports: argument checks only
  EXPECT_RC(gemm_lds_image(P, 100, 64, 2, 0, 32, 128, P, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_lds_image_tile(9, P, 128, 256, 0, 0, P, nullptr), SG_ERR_DTYPE);
  EXPECT_RC(gemm_lds_image_tile(SG_IMG_HALF, P, 128, 256, 0, 64, P, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_lds_image_tile(SG_IMG_FP6, P, 300, 96, 128, 0, P, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_mfma_scale_probe(1, P, P, P, P, P, nullptr), SG_ERR_DTYPE);
  EXPECT_RC(gemm_clock_probe(0, P, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_clock_trace(P, -1, nullptr), SG_ERR_SHAPE);
  EXPECT_RC(gemm_clock_trace(nullptr, 0, nullptr), SG_OK);

  if (std::strlen(gemm_version()) == 0 || gemm_last_error() == nullptr || gemm_last_kernel() == nullptr)
    ++fails;
  if (fails) {
    std::fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  std::puts("C-ABI sanitizer run clean");
  return 0;
}
