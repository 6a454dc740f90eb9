// api.hip -- the C ABI of libswizzled_gemm.so: argument validation, the
// variant plan (tile shape, grid, raster) and the launch on the caller's
// stream.  Every check runs before any HIP call, so each error path is
// reachable on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/swizzled_gemm.h"
#include "launch.h"
#include "lds_layout.h"

namespace {

thread_local std::string g_last_error;
// The clock trace of this thread's launches (gemm_clock_trace); off by default.
thread_local sg::ClockTrace g_clk{nullptr, 0};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SG_OK;
}

int elem_bytes(int dt) {
  switch (dt) {
    case SG_F16:
    case SG_BF16:
      return 2;
    case SG_F32:
      return 4;
    case SG_E4M3:
    case SG_E8M0:
      return 1;
    default:
      return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_out_dtype(int dt) { return dt == SG_F32 || dt == SG_BF16 || dt == SG_F16; }

constexpr int64_t kMaxExtent = (int64_t)1 << 31;  // buffer offsets are 32-bit
constexpr int kCUs = 256;                          // MI355X compute units
constexpr int kGroupM = 8;

// Largest byte extent one workgroup addresses through a buffer resource
// (ld = the operand's leading dimension in elements).
int64_t panel_extent(int major, int64_t rows, int64_t K, int64_t ld, int64_t tile_rows,
                     int eb) {
  if (K == 0) return 0;
  return major == SG_K_MAJOR ? ((rows < tile_rows ? rows : tile_rows) - 1) * ld * eb + K * eb
                             : (K - 1) * ld * eb + rows * eb;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Grouped GEMM and MXFP8: 256x256 tiles when they fill the CUs, or when
// 128x128 tiles would need two or more rounds of the CUs and 256-row panels
// stay within 32-bit buffer offsets (`fits256`); else 128x128 tiles.  Their
// 128x128 kernels trail the 256x256 ping-pongs further than the dense one
// does (MI355X, TFLOP/s 256 vs 128 tiles: MXFP8 2560^3 1176 vs 1014, 3072^3
// 1738 vs 803, 3840^3 2263 vs 1316; grouped bf16 4 x 512 x 4096 x 4096 1055
// vs 1015, 4 x 768 x 4096 x 4096 1345 vs 913), but not one round of them
// (MXFP8 2048^3 755 vs 796).
sg::TileShape pick_tile(int64_t tiles256, int64_t tiles128, bool fits256) {
  if (tiles256 >= kCUs) return sg::kTile256;
  if (fits256 && cdiv(tiles128, kCUs) >= 2) return sg::kTile256;
  return sg::kTile128;
}

// Dense GEMM: 256x256 tiles when they fill the CUs, else 128x128 tiles when
// they fill half of them, else 64x64 tiles (small problems: 1024^3 has 64
// tiles of 128 but 256 of 64).  Between those, when the 256x256 tiles would
// run on the ping-pong (K-major operands, or K a multiple of 64 with two or
// more K tiles) and the 128x128 tiles would need three or more rounds of the
// CUs, one partial round of the ping-pong is faster (bf16 on MI355X, TFLOP/s
// 256 vs 128 tiles: 3072^3 1056 vs 694, 3584^3 1337 vs 911, 3072x3072x1024
// 846 vs 585), though not against one or two rounds of 128x128 tiles
// (2560^3 753 vs 847, 2048x4096x4096 934 vs 1041).
// `fits256`: 256-row panels stay within 32-bit buffer offsets.
sg::TileShape pick_dense_tile(int64_t M, int64_t N, int64_t K, bool a_mn, bool b_mn,
                              bool fits256) {
  if (cdiv(M, 256) * cdiv(N, 256) >= kCUs) return sg::kTile256;
  const int64_t tiles128 = cdiv(M, 128) * cdiv(N, 128);
  const bool pingpong = (!a_mn && !b_mn) || (K % 64 == 0 && K >= 128);
  if (pingpong && fits256 && cdiv(tiles128, kCUs) >= 3) return sg::kTile256;
  if (tiles128 >= kCUs / 2) return sg::kTile128;
  return sg::kTile64;
}

int64_t tile_rows(sg::TileShape t) { return t == sg::kTile256 ? 256 : t == sg::kTile128 ? 128 : 64; }

int hip_fail(hipError_t e, const char* what) {
  return fail(SG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Which kernels dense_run launches.
enum DenseMode { kLibrary, kAblation256, kAblation128, kAblationIO };

// gemm_run, gemm_strided_run, gemm_layout_run and gemm_layout128_run:
// validation, plan and launch.  kLibrary runs the library's kernels; the
// ablation modes run the layout `swz` (16, 8, 0, or padded on 128x128
// tiles) on the 256x256 or 128x128 kernel whatever the problem size.
// Leading dimensions are in elements.
int dense_run(const char* who, DenseMode mode, int swz, int64_t M, int64_t N, int64_t K,
              float alpha,
              const void* A, int64_t lda, int a_major, const void* B, int64_t ldb,
              int b_major, int ab_dtype, float beta, const void* C, int64_t ldc, int c_dtype,
              void* D, int64_t ldd, int d_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 0)
    return fail(SG_ERR_SHAPE, "%s: negative size M=%lld N=%lld K=%lld", who,
                (long long)M, (long long)N, (long long)K);
  if (ab_dtype != SG_F16 && ab_dtype != SG_BF16)
    return fail(SG_ERR_DTYPE, "%s: ab_dtype %d is not SG_F16/SG_BF16", who, ab_dtype);
  if (!is_out_dtype(d_dtype))
    return fail(SG_ERR_DTYPE, "%s: d_dtype %d is not SG_F32/SG_BF16/SG_F16", who, d_dtype);
  if (C && !is_out_dtype(c_dtype))
    return fail(SG_ERR_DTYPE, "%s: c_dtype %d is not SG_F32/SG_BF16/SG_F16", who, c_dtype);
  if (C && C == D && (c_dtype != d_dtype || ldc != ldd))
    return fail(SG_ERR_DTYPE, "%s: in-place C == D needs c_dtype == d_dtype and ldc == ldd",
                who);
  if ((a_major != SG_K_MAJOR && a_major != SG_MN_MAJOR) ||
      (b_major != SG_K_MAJOR && b_major != SG_MN_MAJOR))
    return fail(SG_ERR_MAJOR, "%s: majorness must be SG_K_MAJOR or SG_MN_MAJOR", who);
  if (lda < (a_major == SG_K_MAJOR ? K : M) || ldb < (b_major == SG_K_MAJOR ? K : N) ||
      ldd < N || (C && ldc < N))
    return fail(SG_ERR_SHAPE,
                "%s: a leading dimension is below its minimum (lda %lld, ldb %lld, ldc %lld, "
                "ldd %lld)", who, (long long)lda, (long long)ldb, (long long)ldc,
                (long long)ldd);
  if (N % 4)
    return fail(SG_ERR_SHAPE, "%s: N=%lld is not a multiple of 4 (D is written 4 columns at "
                              "a time)", who, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!D) return fail(SG_ERR_NULL, "%s: D is NULL", who);
  // alpha == 0: A and B are not read; beta == 0: C is not read.
  if (alpha == 0.0f) K = 0;
  if (beta == 0.0f) C = nullptr;
  if (K > 0 && (!A || !B)) return fail(SG_ERR_NULL, "%s: A or B is NULL", who);
  const int eb = 2, db = elem_bytes(d_dtype), cb = C ? elem_bytes(c_dtype) : 0;
  if ((K > 0 && (!aligned16(A) || !aligned16(B))) || !aligned16(D) || (C && !aligned16(C)))
    return fail(SG_ERR_ALIGN, "%s: every pointer must be 16-byte aligned", who);
  if ((K > 0 && ((lda * eb) % 16 || (ldb * eb) % 16)) || (ldd * db) % 16 ||
      (C && (ldc * cb) % 16))
    return fail(SG_ERR_ALIGN,
                "%s: row pitches must be multiples of 16 bytes (A %lld, B %lld, D %lld bytes)",
                who, (long long)(lda * eb), (long long)(ldb * eb), (long long)(ldd * db));
  // The loaders move whole 16-byte chunks of a K-major row: with K % 8 != 0
  // the elements past K in the last chunk would come from the row padding.
  // (Packed rows cannot get here: their pitch 2K is then not a multiple of 16.)
  if (K > 0 && K % 8 && (a_major == SG_K_MAJOR || b_major == SG_K_MAJOR))
    return fail(SG_ERR_SHAPE, "%s: K=%lld is not a multiple of 8 with a K-major operand",
                who, (long long)K);
  const bool fits256 = panel_extent(a_major, M, K, lda, 256, eb) < kMaxExtent &&
                       panel_extent(b_major, N, K, ldb, 256, eb) < kMaxExtent;
  const sg::TileShape tile = mode == kAblation256 || mode == kAblationIO ? sg::kTile256
                            : mode == kAblation128 ? sg::kTile128
                                                   : pick_dense_tile(M, N, K, a_major == SG_MN_MAJOR,
                                                                     b_major == SG_MN_MAJOR,
                                                                     fits256);
  const int64_t T = tile_rows(tile);
  if (panel_extent(a_major, M, K, lda, T, eb) >= kMaxExtent ||
      panel_extent(b_major, N, K, ldb, T, eb) >= kMaxExtent ||
      lda * eb >= kMaxExtent || ldb * eb >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "%s: an operand panel spans 2^31 bytes or more", who);
  const int64_t tiles_m = cdiv(M, T), tiles_n = cdiv(N, T);
  if (tiles_m * tiles_n >= kMaxExtent || tiles_m * tiles_n > 0x7fffffffLL)
    return fail(SG_ERR_SHAPE, "%s: too many tiles", who);

  sg::DenseParams p;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = C ? ldc : 0;
  p.ldd = ldd;
  p.alpha = alpha;
  p.beta = C ? beta : 0.0f;
  p.c_dtype = C ? c_dtype : SG_NONE;
  p.d_dtype = d_dtype;
  p.tiles_m = (int)tiles_m;
  p.tiles_n = (int)tiles_n;
  p.group_m = kGroupM;
  p.clk = g_clk;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = mode == kAblationIO    ? sg::launch_layout_io(swz & 0xff, swz >> 8, p, s)
                       : mode == kAblation256 ? sg::launch_layout(swz, p, s)
                       : mode == kAblation128 ? sg::launch_layout128(swz, p, s)
                                              : sg::launch_dense(tile, ab_dtype == SG_BF16,
                                                                 a_major == SG_MN_MAJOR,
                                                                 b_major == SG_MN_MAJOR, p, s);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

}  // namespace

namespace sg {
const char*& last_kernel() {
  thread_local const char* name = "";
  return name;
}
}  // namespace sg

extern "C" {

const char* gemm_last_kernel(void) { return sg::last_kernel(); }

const char* gemm_last_error(void) { return g_last_error.c_str(); }

const char* gemm_version(void) {
  return "swizzled_gemm 0.3 (gfx950; 16-bit MFMA 16x16x32 and 32x32x16, MXFP8/MXFP6/MXFP4 "
         "scaled MFMA 32x32x64; LDS XOR swizzle over 256-byte bank lines)";
}

int gemm_run(int64_t M, int64_t N, int64_t K, const void* A, int a_major,
             const void* B, int b_major, int ab_dtype, const void* C, int c_dtype,
             void* D, int d_dtype, void* stream) {
  return dense_run("gemm_run", kLibrary, 0, M, N, K, 1.0f, A, a_major == SG_K_MAJOR ? K : M, a_major,
                   B, b_major == SG_K_MAJOR ? K : N, b_major, ab_dtype, 1.0f, C, N, c_dtype,
                   D, N, d_dtype, stream);
}

int gemm_strided_run(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                     int64_t lda, int a_major, const void* B, int64_t ldb, int b_major,
                     int ab_dtype, float beta, const void* C, int64_t ldc, int c_dtype,
                     void* D, int64_t ldd, int d_dtype, void* stream) {
  return dense_run("gemm_strided_run", kLibrary, 0, M, N, K, alpha, A, lda, a_major, B, ldb, b_major,
                   ab_dtype, beta, C, ldc, c_dtype, D, ldd, d_dtype, stream);
}

int gemm_layout_run(int swz_units, int64_t M, int64_t N, int64_t K, const void* A,
                    const void* B, const void* C, int c_dtype, void* D, int d_dtype,
                    void* stream) {
  if (swz_units != 0 && swz_units != 8 && swz_units != 16)
    return fail(SG_ERR_SHAPE, "gemm_layout_run: swz_units %d is not 0, 8 or 16", swz_units);
  return dense_run("gemm_layout_run", kAblation256, swz_units, M, N, K, 1.0f, A, K,
                   SG_K_MAJOR, B, K, SG_K_MAJOR, SG_BF16, 1.0f, C, N, c_dtype, D, N, d_dtype,
                   stream);
}

int gemm_layout_io_run(int operand_swz, int output_swz, int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, const void* C, int c_dtype, void* D,
                       int d_dtype, void* stream) {
  if (operand_swz != 0 && operand_swz != 16)
    return fail(SG_ERR_SHAPE, "gemm_layout_io_run: operand_swz %d is not 0 or 16", operand_swz);
  if (output_swz != 0 && output_swz != 1)
    return fail(SG_ERR_SHAPE, "gemm_layout_io_run: output_swz %d is not 0 or 1", output_swz);
  if (d_dtype != SG_BF16 && d_dtype != SG_F16)
    return fail(SG_ERR_DTYPE, "gemm_layout_io_run: d_dtype %d is not 16-bit (a 16-bit D is "
                              "what the epilogue stages in LDS)", d_dtype);
  if (C && c_dtype != SG_BF16 && c_dtype != SG_F16)
    return fail(SG_ERR_DTYPE, "gemm_layout_io_run: c_dtype %d is not 16-bit", c_dtype);
  return dense_run("gemm_layout_io_run", kAblationIO, operand_swz | (output_swz << 8), M, N, K,
                   1.0f, A, K, SG_K_MAJOR, B, K, SG_K_MAJOR, SG_BF16, 1.0f, C, N, c_dtype, D,
                   N, d_dtype, stream);
}

int gemm_layout128_run(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                       const void* B, const void* C, int c_dtype, void* D, int d_dtype,
                       void* stream) {
  if (layout != 0 && layout != 8 && layout != 16 && layout != SG_LAYOUT_PAD16)
    return fail(SG_ERR_SHAPE, "gemm_layout128_run: layout %d is not 0, 8, 16 or "
                "SG_LAYOUT_PAD16", layout);
  return dense_run("gemm_layout128_run", kAblation128,
                   layout == SG_LAYOUT_PAD16 ? sg::kSwzPad : layout, M, N, K, 1.0f, A, K,
                   SG_K_MAJOR, B, K, SG_K_MAJOR, SG_BF16, 1.0f, C, N, c_dtype, D, N, d_dtype,
                   stream);
}

int grouped_gemm_run(int G, const int64_t* m_offsets, int64_t N, int64_t K,
                     const void* A, int a_major, const void* B, int b_major,
                     int ab_dtype, void* D, int d_dtype, void* stream) {
  if (G < 1 || G > SG_MAX_GROUPS)
    return fail(SG_ERR_GROUPS, "grouped_gemm_run: G=%d outside [1, %d]", G, SG_MAX_GROUPS);
  if (!m_offsets) return fail(SG_ERR_NULL, "grouped_gemm_run: m_offsets is NULL");
  if (m_offsets[0] != 0)
    return fail(SG_ERR_GROUPS, "grouped_gemm_run: m_offsets[0] must be 0");
  for (int g = 0; g < G; ++g)
    if (m_offsets[g + 1] < m_offsets[g])
      return fail(SG_ERR_GROUPS, "grouped_gemm_run: m_offsets decrease at group %d", g);
  if (N < 0 || K < 0)
    return fail(SG_ERR_SHAPE, "grouped_gemm_run: negative size N=%lld K=%lld",
                (long long)N, (long long)K);
  if (ab_dtype != SG_F16 && ab_dtype != SG_BF16)
    return fail(SG_ERR_DTYPE, "grouped_gemm_run: ab_dtype %d is not SG_F16/SG_BF16", ab_dtype);
  if (!is_out_dtype(d_dtype))
    return fail(SG_ERR_DTYPE, "grouped_gemm_run: d_dtype %d unsupported", d_dtype);
  if (a_major != SG_K_MAJOR || b_major != SG_K_MAJOR)
    return fail(SG_ERR_MAJOR, "grouped_gemm_run: A and B must be SG_K_MAJOR");
  const int64_t total = m_offsets[G];
  if (total == 0 || N == 0) return ok();
  if (!D) return fail(SG_ERR_NULL, "grouped_gemm_run: D is NULL");
  if (K > 0 && (!A || !B)) return fail(SG_ERR_NULL, "grouped_gemm_run: A or B is NULL");
  const int eb = 2, db = elem_bytes(d_dtype);
  if ((K > 0 && (!aligned16(A) || !aligned16(B))) || !aligned16(D))
    return fail(SG_ERR_ALIGN, "grouped_gemm_run: every pointer must be 16-byte aligned");
  if ((K * eb) % 16 || (N * db) % 16)
    return fail(SG_ERR_ALIGN, "grouped_gemm_run: row pitches must be multiples of 16 bytes");
  int64_t tiles256 = 0, tiles128 = 0;
  for (int g = 0; g < G; ++g) {
    tiles256 += cdiv(m_offsets[g + 1] - m_offsets[g], 256);
    tiles128 += cdiv(m_offsets[g + 1] - m_offsets[g], 128);
  }
  tiles256 *= cdiv(N, 256);
  tiles128 *= cdiv(N, 128);
  const sg::TileShape tile = pick_tile(tiles256, tiles128, 256 * K * eb < kMaxExtent);
  const int64_t T = tile == sg::kTile256 ? 256 : 128;
  if (T * K * eb >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "grouped_gemm_run: an operand panel spans 2^31 bytes or more");
  sg::GroupedParams p;
  p.A = A;
  p.B = B;
  p.D = D;
  p.N = N;
  p.K = K;
  p.d_dtype = d_dtype;
  p.G = G;
  p.tiles_n = (int)cdiv(N, T);
  p.group_m = kGroupM;
  p.clk = g_clk;
  int64_t acc = 0;
  for (int g = 0; g <= G; ++g) {
    p.m_off[g] = m_offsets[g];
    p.tile_start[g] = (int32_t)acc;
    if (g < G) acc += cdiv(m_offsets[g + 1] - m_offsets[g], T) * p.tiles_n;
    if (acc > 0x7fffffffLL) return fail(SG_ERR_SHAPE, "grouped_gemm_run: too many tiles");
  }
  for (int g = G + 1; g <= SG_MAX_GROUPS; ++g) {
    p.m_off[g] = m_offsets[G];
    p.tile_start[g] = (int32_t)acc;
  }
  if (acc == 0) return ok();
  hipError_t e = sg::launch_grouped(tile, ab_dtype == SG_BF16, sg::kSwzDefault, p,
                                    (int)acc, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "grouped_gemm_run launch");
  return ok();
}

namespace {

// The shared checks and launch of the block-scaled GEMMs: fmt SG_E4M3,
// SG_E2M1, SG_E2M3 or SG_E3M2; scales in layout sf_layout (SG_SF_ROWS: 4-byte
// aligned; SG_SF_BLOCKS: 16-byte aligned).
int mx_run(const char* who, int fmt, int sf_layout, int64_t M, int64_t N, int64_t K,
           const void* A, const void* SFA, const void* B, const void* SFB, void* D,
           int d_dtype, void* stream) {
  const bool fp4 = fmt == SG_E2M1, fp6 = fmt == SG_E2M3 || fmt == SG_E3M2;
  if (fmt != SG_E4M3 && !fp4 && !fp6)
    return fail(SG_ERR_DTYPE, "%s: fmt %d is not SG_E4M3/SG_E2M1/SG_E2M3/SG_E3M2", who, fmt);
  if (sf_layout != SG_SF_ROWS && sf_layout != SG_SF_BLOCKS)
    return fail(SG_ERR_SHAPE, "%s: sf_layout %d is not SG_SF_ROWS/SG_SF_BLOCKS", who, sf_layout);
  if (M < 0 || N < 0 || K < 0) return fail(SG_ERR_SHAPE, "%s: negative size", who);
  const int64_t kmul = fp4 ? 256 : 128;
  if (K % kmul)
    return fail(SG_ERR_SHAPE, "%s: K=%lld is not a multiple of %lld", who, (long long)K,
                (long long)kmul);
  if (d_dtype != SG_F32 && d_dtype != SG_BF16)
    return fail(SG_ERR_DTYPE, "%s: d_dtype %d is not SG_F32/SG_BF16", who, d_dtype);
  if (M == 0 || N == 0) return ok();
  if (!D) return fail(SG_ERR_NULL, "%s: D is NULL", who);
  if (K > 0 && (!A || !B || !SFA || !SFB))
    return fail(SG_ERR_NULL, "%s: A, B, SFA or SFB is NULL", who);
  const int db = elem_bytes(d_dtype);
  const uintptr_t sf_mask = sf_layout == SG_SF_BLOCKS ? 15u : 3u;
  if ((K > 0 && (!aligned16(A) || !aligned16(B))) || !aligned16(D) ||
      (K > 0 && ((reinterpret_cast<uintptr_t>(SFA) | reinterpret_cast<uintptr_t>(SFB)) & sf_mask)))
    return fail(SG_ERR_ALIGN, "%s: A, B, D must be 16-byte aligned, SFA and SFB %d-byte aligned",
                who, sf_layout == SG_SF_BLOCKS ? 16 : 4);
  if ((N * db) % 16)
    return fail(SG_ERR_ALIGN, "%s: D row pitch must be a multiple of 16 bytes", who);
  // MXFP8 takes 128x128 tiles for small problems; the others 256x256.
  const int64_t row_bytes = fp4 ? K / 2 : fp6 ? K / 4 * 3 : K;
  const bool fits256 = 256 * row_bytes < kMaxExtent &&
                       (sf_layout != SG_SF_BLOCKS || 4 * cdiv(K, 512) * 1024 < kMaxExtent);
  const sg::TileShape tile =
      fmt == SG_E4M3 ? pick_tile(cdiv(M, 256) * cdiv(N, 256), cdiv(M, 128) * cdiv(N, 128), fits256)
                     : sg::kTile256;
  const int64_t T = tile == sg::kTile256 ? 256 : 128;
  // a tile's panel (plus, for fp6, the 8 bytes its shifted rows may read beyond it)
  if (T * row_bytes + (fp6 ? 8 : 0) >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "%s: an operand panel spans 2^31 bytes or more", who);
  if (sf_layout == SG_SF_BLOCKS && cdiv(T, 64) * cdiv(K, 512) * 1024 >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "%s: a tile's scales span 2^31 bytes or more", who);
  const int64_t tiles_m = cdiv(M, T), tiles_n = cdiv(N, T);
  if (tiles_m * tiles_n > 0x7fffffffLL) return fail(SG_ERR_SHAPE, "%s: too many tiles", who);
  sg::MxParams p;
  p.A = A;
  p.SFA = SFA;
  p.B = B;
  p.SFB = SFB;
  p.D = D;
  p.M = M;
  p.N = N;
  p.K = K;
  p.d_dtype = d_dtype;
  p.sf_layout = sf_layout;
  p.tiles_m = (int)tiles_m;
  p.tiles_n = (int)tiles_n;
  p.group_m = kGroupM;
  p.clk = g_clk;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fp4   ? sg::launch_mxfp4(p, s)
                       : fp6 ? sg::launch_mxfp6(fmt == SG_E3M2, p, s)
                             : sg::launch_mx(tile, p, s);
  if (e != hipSuccess) return fail(SG_ERR_HIP, "%s launch: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

int mxfp4_gemm_run(int64_t M, int64_t N, int64_t K, const void* A, const void* SFA,
                   const void* B, const void* SFB, void* D, int d_dtype, void* stream) {
  return mx_run("mxfp4_gemm_run", SG_E2M1, SG_SF_ROWS, M, N, K, A, SFA, B, SFB, D, d_dtype,
                stream);
}

int mxfp6_gemm_run(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* SFA,
                   const void* B, const void* SFB, void* D, int d_dtype, void* stream) {
  if (fmt != SG_E2M3 && fmt != SG_E3M2)
    return fail(SG_ERR_DTYPE, "mxfp6_gemm_run: fmt %d is not SG_E2M3/SG_E3M2", fmt);
  return mx_run("mxfp6_gemm_run", fmt, SG_SF_ROWS, M, N, K, A, SFA, B, SFB, D, d_dtype, stream);
}

int mx_gemm_run(int64_t M, int64_t N, int64_t K, const void* A, const void* SFA,
                const void* B, const void* SFB, void* D, int d_dtype, void* stream) {
  return mx_run("mx_gemm_run", SG_E4M3, SG_SF_ROWS, M, N, K, A, SFA, B, SFB, D, d_dtype,
                stream);
}

int mx_gemm_blocks_run(int fmt, int64_t M, int64_t N, int64_t K, const void* A,
                       const void* SFA, const void* B, const void* SFB, void* D, int d_dtype,
                       void* stream) {
  return mx_run("mx_gemm_blocks_run", fmt, SG_SF_BLOCKS, M, N, K, A, SFA, B, SFB, D, d_dtype,
                stream);
}

int64_t mx_scales_blocks_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || K % 32)
    return fail(SG_ERR_SHAPE, "mx_scales_blocks_bytes: rows=%lld K=%lld (K a multiple of 32)",
                (long long)rows, (long long)K);
  return cdiv(rows, 64) * cdiv(K, 512) * 1024;
}

int mx_scales_to_blocks(const void* SF, int64_t rows, int64_t K, void* out, void* stream) {
  if (rows < 0 || K < 0 || K % 128)
    return fail(SG_ERR_SHAPE, "mx_scales_to_blocks: rows=%lld K=%lld (K a multiple of 128)",
                (long long)rows, (long long)K);
  if (rows == 0 || K == 0) return ok();
  if (!SF || !out) return fail(SG_ERR_NULL, "mx_scales_to_blocks: SF or out is NULL");
  if ((reinterpret_cast<uintptr_t>(SF) & 3u) || !aligned16(out))
    return fail(SG_ERR_ALIGN, "mx_scales_to_blocks: SF must be 4-byte, out 16-byte aligned");
  if (cdiv(rows, 64) > 0x7fffffffLL || cdiv(cdiv(K, 512), 16) > 65535)
    return fail(SG_ERR_SHAPE, "mx_scales_to_blocks: too many rows or K blocks");
  hipError_t e = sg::launch_sf_blocks(SF, rows, K, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_scales_to_blocks launch");
  return ok();
}

int gemm_clock_trace(void* buf, int64_t slots, int* wall_khz) {
  if (slots < 0) return fail(SG_ERR_SHAPE, "gemm_clock_trace: slots=%lld < 0", (long long)slots);
  if (buf && (reinterpret_cast<uintptr_t>(buf) & 7u))
    return fail(SG_ERR_ALIGN, "gemm_clock_trace: buf must be 8-byte aligned");
  if (wall_khz) {
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return hip_fail(e, "gemm_clock_trace: wall clock rate");
    *wall_khz = khz;
  }
  g_clk.buf = static_cast<uint64_t*>(buf);
  g_clk.slots = buf ? slots : 0;
  return ok();
}

int gemm_clock_probe(int64_t iters, void* out, void* stream) {
  if (!out) return fail(SG_ERR_NULL, "gemm_clock_probe: out is NULL");
  if (reinterpret_cast<uintptr_t>(out) & 7u)
    return fail(SG_ERR_ALIGN, "gemm_clock_probe: out must be 8-byte aligned");
  if (iters < 1 || iters > (int64_t{1} << 24))
    return fail(SG_ERR_SHAPE, "gemm_clock_probe: iters=%lld outside [1, 2^24]",
                (long long)iters);
  hipError_t e = sg::launch_clock_probe(iters, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_clock_probe launch");
  return ok();
}

int gemm_clock_probe_waves(void) { return sg::clock_probe_waves(); }

int gemm_lds_layout(int rows, int row_bytes, int32_t* out) {
  if (!out) return fail(SG_ERR_NULL, "gemm_lds_layout: out is NULL");
  if (rows <= 0 || rows % 8 || (row_bytes != 64 && row_bytes != 128 && row_bytes != 256))
    return fail(SG_ERR_SHAPE, "gemm_lds_layout: rows must be a positive multiple of 8 "
                              "and row_bytes 64, 128 or 256");
  const int chunks = row_bytes / 16;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < chunks; ++c)
      out[r * chunks + c] = (int32_t)sg::lds_offset_rt(row_bytes, sg::kSwzDefault, r, c);
  return ok();
}

int gemm_lds_layout_mxfp6(int rows, int unshifted, int32_t* out) {
  if (!out) return fail(SG_ERR_NULL, "gemm_lds_layout_mxfp6: out is NULL");
  if (rows <= 0 || rows % 32 || unshifted < 0 || unshifted > 32)
    return fail(SG_ERR_SHAPE, "gemm_lds_layout_mxfp6: rows must be a positive multiple of 32 "
                              "and unshifted in [0, 32]");
  for (int r = 0; r < rows; ++r)
    for (int q = 0; q < 12; ++q)
      out[r * 12 + q] = (int32_t)sg::mxfp6_lds_offset(r, 8u * q, (uint32_t)unshifted);
  return ok();
}

int gemm_lds_layout_cblock(int32_t* out) {
  if (!out) return fail(SG_ERR_NULL, "gemm_lds_layout_cblock: out is NULL");
  for (int w = 0; w < 4; ++w)
    for (int r = 0; r < 128; ++r)
      for (int c = 0; c < 8; ++c)
        out[(w * 128 + r) * 8 + c] = (int32_t)sg::cblock_lds_offset(w, r, c);
  return ok();
}

int gemm_lds_image_tile(int kind, const void* X, int64_t rows, int64_t row_bytes,
                        int64_t row0, int64_t byte0, void* out, void* stream) {
  const char* who = "gemm_lds_image_tile";
  if (kind < SG_IMG_HALF || kind > SG_IMG_CBLOCK)
    return fail(SG_ERR_DTYPE, "%s: unknown kind %d", who, kind);
  if (!X || !out) return fail(SG_ERR_NULL, "%s: X or out is NULL", who);
  if (!aligned16(X) || !aligned16(out) || row_bytes % 16)
    return fail(SG_ERR_ALIGN, "%s: X and out must be 16-byte aligned and row_bytes a "
                              "multiple of 16", who);
  if (rows <= 0 || row_bytes <= 0 || row0 < 0 || row0 >= rows || byte0 < 0 ||
      byte0 >= row_bytes || rows * row_bytes >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "%s: origin (%lld, %lld) outside the %lld x %lld operand", who,
                (long long)row0, (long long)byte0, (long long)rows, (long long)row_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const char* x = static_cast<const char*>(X);
  hipError_t e = hipSuccess;
  if (kind == SG_IMG_HALF || kind == SG_IMG_HALF_KEXACT) {
    if (byte0 % 128 || (kind == SG_IMG_HALF_KEXACT && row_bytes % 128))
      return fail(SG_ERR_SHAPE, "%s: byte0 %% 128 and (K-exact) row_bytes %% 128 must be 0",
                  who);
    const int64_t valid = rows - row0;
    e = sg::launch_lds_image_pp(kind, x + row0 * row_bytes, (uint32_t)(valid * row_bytes),
                                (uint32_t)row_bytes, (int)(valid < 256 ? valid : 256),
                                (uint32_t)byte0, (uint32_t)row_bytes, 32u, 0u, out, s);
  } else if (kind == SG_IMG_MN256) {
    if (row0 % 64 || byte0 % 256)
      return fail(SG_ERR_SHAPE, "%s: row0 %% 64 and byte0 %% 256 must be 0", who);
    const int64_t cols = (row_bytes - byte0) / 2;
    e = sg::launch_lds_image_pp(kind, x + byte0,
                                (uint32_t)((rows - 1) * row_bytes + (row_bytes - byte0)),
                                (uint32_t)row_bytes, (int)(cols < 256 ? cols : 256), 0u, 0u,
                                32u, (uint32_t)(row0 / 64), out, s);
  } else if (kind == SG_IMG_FP6) {
    if (row0 % 256 || byte0 % 96 || row_bytes % 96)
      return fail(SG_ERR_SHAPE, "%s: row0 %% 256, byte0 %% 96 and row_bytes %% 96 must be 0",
                  who);
    // As the MX kernel sets up a 256-row tile: below the operand's last tile
    // the descriptor covers the 8 bytes its shifted rows read past the tile;
    // in the last tile the rows at the last row's block position stay
    // unshifted.
    const int64_t left = rows - row0;
    const int m_valid = (int)(left < 256 ? left : 256);
    const uint32_t bytes = (uint32_t)(m_valid * row_bytes) + (left > 256 ? 8u : 0u);
    const uint32_t unshifted = left > 256 ? 32u : (uint32_t)((left - 1) & 31);
    e = sg::launch_lds_image_pp(kind, x + row0 * row_bytes, bytes, (uint32_t)row_bytes,
                                m_valid, 0u, 0u, unshifted, (uint32_t)(byte0 / 96), out, s);
  } else {
    if (row0 % 256 || byte0 % 512 || row_bytes / 2 > (int64_t{1} << 22))
      return fail(SG_ERR_SHAPE, "%s: row0 %% 256 and byte0 %% 512 must be 0 (and ldc <= "
                  "2^22)", who);
    const int64_t left = rows - row0, cols = (row_bytes - byte0) / 2;
    e = sg::launch_lds_image_cblock(X, row_bytes / 2, row0, byte0 / 2,
                                    (int)(left < 256 ? left : 256),
                                    (int)(cols < 256 ? cols : 256), out, s);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int gemm_mfma_scale_probe(int fmt, const void* a, const void* b, const void* sa,
                          const void* sb, void* out, void* stream) {
  if (fmt != 0 && fmt != 2 && fmt != 3 && fmt != 4)
    return fail(SG_ERR_DTYPE, "gemm_mfma_scale_probe: fmt %d is not 0, 2, 3 or 4", fmt);
  if (!a || !b || !sa || !sb || !out)
    return fail(SG_ERR_NULL, "gemm_mfma_scale_probe: a NULL pointer");
  if (!aligned16(a) || !aligned16(b) || !aligned16(out))
    return fail(SG_ERR_ALIGN, "gemm_mfma_scale_probe: a, b and out must be 16-byte aligned");
  hipError_t e = sg::launch_mfma_scale_probe(fmt, a, b, sa, sb, out,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_mfma_scale_probe launch");
  return ok();
}

int gemm_lds_image(const void* X, int64_t rows_total, int64_t K, int elem_bytes_,
                   int64_t row0, int64_t k0, int tile_rows, void* out, void* stream) {
  if (!X || !out) return fail(SG_ERR_NULL, "gemm_lds_image: X or out is NULL");
  if (elem_bytes_ != 1 && elem_bytes_ != 2)
    return fail(SG_ERR_DTYPE, "gemm_lds_image: elem_bytes must be 1 or 2");
  if (tile_rows != 128 && tile_rows != 256)
    return fail(SG_ERR_SHAPE, "gemm_lds_image: tile_rows must be 128 or 256");
  if (rows_total < 0 || K <= 0 || row0 < 0 || row0 >= rows_total || k0 < 0 || k0 >= K ||
      (k0 * elem_bytes_) % 128)
    return fail(SG_ERR_SHAPE, "gemm_lds_image: tile origin out of range or not on a "
                              "128-byte K boundary");
  if (!aligned16(X) || !aligned16(out) || (K * elem_bytes_) % 16)
    return fail(SG_ERR_ALIGN, "gemm_lds_image: 16-byte alignment required");
  if ((int64_t)tile_rows * K * elem_bytes_ >= kMaxExtent)
    return fail(SG_ERR_SHAPE, "gemm_lds_image: panel spans 2^31 bytes or more");
  hipError_t e = sg::launch_lds_image(X, rows_total, K, elem_bytes_, row0, k0, tile_rows,
                                      out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_lds_image launch");
  return ok();
}

}  // extern "C"
