/*
 * swizzled_gemm.h -- C ABI of libswizzled_gemm.so, an MI355X (gfx950) GEMM
 * whose operand tiles are staged in LDS under an XOR swizzle.
 *
 * Operation.  D = A*B (+C): a tiled matrix multiply-accumulate with 16-bit
 * inputs and fp32 accumulation -- the tensor-core operation D = A*B + C of
 * "Tensor Cores, layouts, and swizzling" (opening section), computed by the
 * sample tiled matmul of "Swizzling explained properly" (section "Sample
 * swizzled matmul") with tiles staged in on-chip memory under the swizzle
 * f(r, c) = (r, c XOR r) of that page (section "What does swizzling do?").
 * Passing C = NULL computes D = A*B, the "enable-input-d = false" form of
 * "06 Blackwell Tensor Core - tcgen05 MMA" (operand table); a non-NULL C is
 * the accumulate form D = A*B + C.
 *
 * Conventions shared by every entry point:
 *  - All pointers named A, B, C, D, SFA, SFB are DEVICE pointers of the
 *    current HIP device; m_offsets is a HOST pointer.  The caller owns every
 *    buffer; the library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *    call enqueues its kernels on that stream and returns at once; results
 *    are visible after the stream is synchronised.
 *  - Matrices are dense and row-major with no padding: a "K-major" operand
 *    is stored [rows][K] (K contiguous), an "MN-major" one [K][rows].
 *    A: K-major [M][K] or MN-major [K][M].  B: K-major [N][K] (B transposed)
 *    or MN-major [K][N].  C and D: [M][N].
 *  - Every pointer must be 16-byte aligned and every row pitch (contiguous
 *    extent x element size) a multiple of 16 bytes, the 16-byte atom rule of
 *    both swizzle pages ("LBO, SBO and SWZ", section 1; "Swizzling explained
 *    properly", section "What about base?") and of the TMA stride rule in
 *    "Tensor Cores, layouts, and swizzling".  Violations return
 *    SG_ERR_ALIGN.  M, N and K themselves may be ragged (not multiples of
 *    the tile); M = 0 or N = 0 is a no-op; K = 0 gives D = C (or 0).
 *  - Return value: SG_OK (0) or a negative SG_ERR_* code; on error nothing is
 *    enqueued and gemm_last_error() describes the failure (thread-local).
 */
#ifndef SWIZZLED_GEMM_H
#define SWIZZLED_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SG_OK 0
#define SG_ERR_NULL (-1)   /* a required pointer is NULL */
#define SG_ERR_ALIGN (-2)  /* pointer not 16-byte aligned, or row pitch not a multiple of 16 B */
#define SG_ERR_SHAPE (-3)  /* negative size, or beyond the supported extent */
#define SG_ERR_DTYPE (-4)  /* unsupported element type combination */
#define SG_ERR_MAJOR (-5)  /* majorness not SG_K_MAJOR / SG_MN_MAJOR */
#define SG_ERR_GROUPS (-6) /* bad group count or offsets */
#define SG_ERR_HIP (-7)    /* a HIP call failed; see gemm_last_error() */

/* Element types. */
#define SG_NONE 0
#define SG_F16 1  /* IEEE binary16 */
#define SG_BF16 2 /* bfloat16 */
#define SG_F32 3  /* IEEE binary32 */
#define SG_E4M3 4 /* OCP FP8 E4M3 (bias 7, max 448, no infinity) */
#define SG_E8M0 5 /* OCP E8M0 scale, value 2^(e-127) */
#define SG_E2M1 6 /* OCP FP4 E2M1 (bias 1, max 6, two elements per byte) */
#define SG_E2M3 7 /* OCP FP6 E2M3 (bias 1, max 7.5, no infinity or NaN) */
#define SG_E3M2 8 /* OCP FP6 E3M2 (bias 3, max 28, no infinity or NaN) */

/* Layouts of the e8m0 scale arrays of the block-scaled GEMMs. */
#define SG_SF_ROWS 0   /* [rows][K/32]: row r's byte b at r * (K/32) + b */
#define SG_SF_BLOCKS 1 /* 1 KiB blocks of 64 rows x 16 bytes, see mx_scales_to_blocks */

/* Operand majorness. */
#define SG_K_MAJOR 0  /* K is the contiguous dimension */
#define SG_MN_MAJOR 1 /* M (for A) or N (for B) is the contiguous dimension */

/* Largest group count grouped_gemm_run accepts. */
#define SG_MAX_GROUPS 256

/*
 * gemm_run -- D = A*B (+C), fp32 accumulation.
 *   M, N, K    problem sizes (>= 0).
 *   A          ab_dtype, K-major [M][K] or MN-major [K][M] (a_major).
 *   B          ab_dtype, K-major [N][K] or MN-major [K][N] (b_major).
 *   ab_dtype   SG_F16 or SG_BF16.
 *   C          NULL (treated as zero) or [M][N] of c_dtype (SG_F32, SG_BF16,
 *              SG_F16).  C may equal D (in-place accumulate) when c_dtype ==
 *              d_dtype; any other overlap of C or D with inputs is undefined.
 *   D          [M][N] of d_dtype: SG_F32, SG_BF16 or SG_F16 (the fp32
 *              accumulator is rounded to nearest even).
 * Errors: SG_ERR_NULL (A, B or D NULL with M, N > 0 -- A/B may be NULL when
 * K = 0), SG_ERR_ALIGN, SG_ERR_SHAPE (a size < 0, or a per-tile operand
 * extent of 2^31 bytes or more), SG_ERR_DTYPE, SG_ERR_MAJOR, SG_ERR_HIP.
 */
int gemm_run(int64_t M, int64_t N, int64_t K, const void* A, int a_major,
             const void* B, int b_major, int ab_dtype, const void* C,
             int c_dtype, void* D, int d_dtype, void* stream);

/*
 * gemm_strided_run -- D = alpha * A*B + beta * C with leading dimensions,
 * fp32 accumulation.  Operands are addressed as "Tensor Cores, layouts, and
 * swizzling" describes its tensor-memory tile copies (section on the Tensor
 * Memory Accelerator): by dimensions and row strides that are multiples of
 * 16 bytes, with elements past the edges read as zero.
 *   alpha, beta  fp32 scalars.  D = round(alpha * acc + beta * C) with acc the
 *                fp32 sum over K; alpha = beta = 1 gives gemm_run's result
 *                bit for bit.  alpha == 0: A and B are not read (D = beta*C);
 *                beta == 0 or C == NULL: C is not read.
 *   A   K-major: element (m, k) at A[m*lda + k], lda >= K;
 *       MN-major: element (m, k) at A[k*lda + m], lda >= M.
 *   B   K-major: element (k, n) at B[n*ldb + k], ldb >= K;
 *       MN-major: element (k, n) at B[k*ldb + n], ldb >= N.
 *   C   element (m, n) at C[m*ldc + n], ldc >= N; D at D[m*ldd + n], ldd >= N.
 *   Leading dimensions are in elements; every row pitch (ld * element size)
 *   must be a multiple of 16 bytes and every pointer 16-byte aligned.  C may
 *   equal D when c_dtype == d_dtype and ldc == ldd.  The other arguments and
 *   the errors are gemm_run's, plus SG_ERR_SHAPE for a leading dimension below
 *   its minimum, an N that is not a multiple of 4 (the epilogue writes D
 *   four columns at a time; gemm_run's packed rows already imply it), or a
 *   K that is not a multiple of 8 while A or B is K-major (the loaders move
 *   whole 16-byte chunks of a row, so the elements past K inside the last
 *   chunk would be read from the row's padding; gemm_run's packed K-major
 *   rows already imply K % 8 == 0 through the 16-byte pitch rule).
 */
int gemm_strided_run(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                     int64_t lda, int a_major, const void* B, int64_t ldb, int b_major,
                     int ab_dtype, float beta, const void* C, int64_t ldc, int c_dtype,
                     void* D, int64_t ldd, int d_dtype, void* stream);

/*
 * grouped_gemm_run -- for each group g in [0, G):
 *   D[off_g : off_{g+1}] = A[off_g : off_{g+1}] * B_g,
 * the grouped GEMM named in "LBO, SBO and SWZ for a tcgen05 tile"
 * (introduction); the pages give no further definition, so each group is the
 * plain dense GEMM on its row range.  Groups share N and K.
 *   G          number of groups, 1..SG_MAX_GROUPS.
 *   m_offsets  HOST array of G+1 row offsets: m_offsets[0] = 0, non-
 *              decreasing; group g owns rows [m_offsets[g], m_offsets[g+1]).
 *              Empty groups are allowed.  Read during the call only.
 *   A          ab_dtype, K-major [m_offsets[G]][K].
 *   B          ab_dtype, G contiguous blocks, each K-major [N][K]
 *              (b_major must be SG_K_MAJOR).
 *   D          [m_offsets[G]][N] of d_dtype (SG_F32, SG_BF16, SG_F16).
 * Errors: as gemm_run, plus SG_ERR_GROUPS (G out of range, m_offsets[0] != 0
 * or decreasing offsets).
 */
int grouped_gemm_run(int G, const int64_t* m_offsets, int64_t N, int64_t K,
                     const void* A, int a_major, const void* B, int b_major,
                     int ab_dtype, void* D, int d_dtype, void* stream);

/*
 * mx_gemm_run -- block-scaled (MXFP8) GEMM:
 *   D[m][n] = sum_blk 2^(SFA[m][blk]-127) * 2^(SFB[n][blk]-127)
 *             * sum_{k in blk} A[m][k] * B[n][k],
 * with 32-element K blocks: output (m, n) uses SFA[m, sfk] for A and
 * SFB[n, sfk] for B ("06 Blackwell Tensor Core - tcgen05 MMA", section
 * "Block-Scaled MMA").  fp32 accumulation.
 *   A    e4m3 K-major [M][K];  SFA  e8m0 [M][K/32].
 *   B    e4m3 K-major [N][K];  SFB  e8m0 [N][K/32].
 *   D    [M][N] of d_dtype (SG_F32 or SG_BF16).
 *   K    must be a multiple of 128 (four scale blocks per 16-byte row chunk
 *        pair); M and N may be ragged.
 * Scale byte 255 (NaN) propagates NaN.
 * Errors: SG_ERR_NULL, SG_ERR_ALIGN, SG_ERR_SHAPE (K % 128 != 0 or extents),
 * SG_ERR_DTYPE, SG_ERR_HIP.
 */
int mx_gemm_run(int64_t M, int64_t N, int64_t K, const void* A,
                const void* SFA, const void* B, const void* SFB, void* D,
                int d_dtype, void* stream);

/*
 * mxfp4_gemm_run -- the block-scaled GEMM of mx_gemm_run with OCP FP4 E2M1
 * elements (MXFP4): 1 sign, 2 exponent bits (bias 1), 1 fraction bit,
 * values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; two elements per byte, element 2i
 * in the low nibble of byte i.  The scale rule is mx_gemm_run's ("06
 * Blackwell Tensor Core - tcgen05 MMA", section "Block-Scaled MMA"); the
 * 32-element block and e8m0 scales as there.  fp32 accumulation.
 *   A    e2m1 K-major [M][K/2] bytes;  SFA  e8m0 [M][K/32].
 *   B    e2m1 K-major [N][K/2] bytes;  SFB  e8m0 [N][K/32].
 *   D    [M][N] of d_dtype (SG_F32 or SG_BF16).
 *   K    must be a multiple of 256 (one 128-byte row chunk per K tile);
 *        M and N may be ragged.
 * Errors: SG_ERR_NULL, SG_ERR_ALIGN, SG_ERR_SHAPE (K % 256 != 0 or
 * extents), SG_ERR_DTYPE, SG_ERR_HIP.
 */
int mxfp4_gemm_run(int64_t M, int64_t N, int64_t K, const void* A,
                   const void* SFA, const void* B, const void* SFB, void* D,
                   int d_dtype, void* stream);

/*
 * mxfp6_gemm_run -- the block-scaled GEMM of mx_gemm_run with OCP FP6
 * elements (MXFP6): fmt SG_E2M3 (1 sign, 2 exponent bits with bias 1, 3
 * fraction bits; largest magnitude 7.5, smallest 0.125) or SG_E3M2 (1 sign,
 * 3 exponent bits with bias 3, 2 fraction bits; largest 28, smallest
 * 0.0625); neither has infinity or NaN.  A row is a 6-bit stream: element k
 * at bits [6k, 6k+6) of the row's bytes, little endian (four elements in
 * three bytes).  The scale rule is mx_gemm_run's ("06 Blackwell Tensor Core
 * - tcgen05 MMA", section "Block-Scaled MMA"); the 32-element block and
 * e8m0 scales as there.  fp32 accumulation.
 *   A    fp6 K-major [M][3K/4] bytes;  SFA  e8m0 [M][K/32].
 *   B    fp6 K-major [N][3K/4] bytes;  SFB  e8m0 [N][K/32].
 *   D    [M][N] of d_dtype (SG_F32 or SG_BF16).
 *   K    must be a multiple of 128 (96 bytes of every row per K tile);
 *        M and N may be ragged.  No read leaves the M*3K/4 bytes of A, the
 *        N*3K/4 bytes of B or the scale arrays.
 * Errors: SG_ERR_NULL, SG_ERR_ALIGN, SG_ERR_SHAPE (K % 128 != 0 or
 * extents), SG_ERR_DTYPE (fmt or d_dtype), SG_ERR_HIP.
 */
int mxfp6_gemm_run(int fmt, int64_t M, int64_t N, int64_t K, const void* A,
                   const void* SFA, const void* B, const void* SFB, void* D,
                   int d_dtype, void* stream);

/*
 * mx_scales_blocks_bytes -- the size in bytes of an e8m0 scale array of
 * `rows` rows and K/32 blocks in the SG_SF_BLOCKS layout (host-side, no GPU
 * needed): ceil(rows/64) * ceil(K/512) * 1024.  Returns SG_ERR_SHAPE
 * (negative) for rows < 0, K < 0 or K not a multiple of 32.
 */
int64_t mx_scales_blocks_bytes(int64_t rows, int64_t K);

/*
 * mx_scales_to_blocks -- rearranges e8m0 scales SF [rows][K/32] (SG_SF_ROWS,
 * the layout of "06 Blackwell Tensor Core - tcgen05 MMA", section
 * "Block-Scaled MMA": SFA(M, SFK), SFB(N, SFK)) into `out`, SG_SF_BLOCKS:
 * row r's scale byte b (32-element block b of K) goes to byte
 *   ((r / 64) * G + b / 16) * 1024 + (r % 64) * 16 + 8 * (b % 2) + (b % 16) / 2,
 * G = ceil(K/512): the 16 bytes of one group of 16 blocks for 64 consecutive
 * rows are one contiguous KiB, and a row's 16 bytes hold the group's 8 even
 * blocks, then its 8 odd ones.  Bytes for rows past `rows` (up to the next
 * multiple of 64) and blocks past K/32 are written as zero.  The scaled
 * MFMA's two lane halves scale the even and the odd blocks of a 64-wide K
 * step, so the block-scaled GEMMs load a row's group as one 8-byte half per
 * lane, with no rearranging after the load; from SG_SF_BLOCKS a wave's load
 * of 32 rows covers 4 cache lines instead of the 32 (one per row) of
 * SG_SF_ROWS.  SF: DEVICE memory, 4-byte aligned; out: DEVICE memory of
 * mx_scales_blocks_bytes(rows, K) bytes, 16-byte aligned (caller-owned).
 * Asynchronous on `stream` (a hipStream_t, NULL for the default stream).
 * Errors: SG_ERR_SHAPE (K not a multiple of 128, negative sizes, 2^31 or
 * more blocks of 64 rows, K past 2^29), SG_ERR_NULL, SG_ERR_ALIGN,
 * SG_ERR_HIP.
 */
int mx_scales_to_blocks(const void* SF, int64_t rows, int64_t K, void* out, void* stream);

/*
 * mx_gemm_blocks_run -- the block-scaled GEMM of mx_gemm_run (fmt SG_E4M3),
 * mxfp4_gemm_run (SG_E2M1) or mxfp6_gemm_run (SG_E2M3, SG_E3M2), with SFA
 * and SFB in the SG_SF_BLOCKS layout (mx_scales_to_blocks), 16-byte aligned.
 * The layout's padding (rows past M or N in the last 64 rows, blocks past
 * K/32 in the last group) is never used and may hold anything.  Every other
 * argument, requirement and result is that entry point's; the D it computes
 * is bit-identical.  Errors: theirs, and SG_ERR_DTYPE for
 * another fmt.
 */
int mx_gemm_blocks_run(int fmt, int64_t M, int64_t N, int64_t K, const void* A,
                       const void* SFA, const void* B, const void* SFB, void* D,
                       int d_dtype, void* stream);

/*
 * gemm_layout_run -- the bf16 GEMM with A and B K-major (and optional C) on
 * 256x256 tiles of the 8-wave ping-pong kernel with 32x32x16 MFMAs (the
 * 16x16x32 variant of gemm_run reads fragments in another lane pattern), with
 * a chosen LDS operand layout: the layout experiment of "Swizzling explained
 * properly" (sections "Why swizzle?" and "Results") on gfx950.
 *   swz_units  16: the library's layout (the 16-byte unit index XORed with
 *              the 256-byte bank-line index: ds_read_b128 reads 64 banks of
 *              4 bytes); 8: the same XOR over 128-byte lines; 0: no swizzle.
 * Every layout gives the same D; only LDS bank conflicts and speed differ.
 * The other arguments are gemm_run's (ab_dtype = SG_BF16, both operands
 * SG_K_MAJOR).  Errors: as gemm_run, and SG_ERR_SHAPE for swz_units not in
 * {0, 8, 16}.
 */
int gemm_layout_run(int swz_units, int64_t M, int64_t N, int64_t K, const void* A,
                    const void* B, const void* C, int c_dtype, void* D, int d_dtype,
                    void* stream);

/*
 * gemm_layout_io_run -- the input/output half of the layout experiment of
 * "Swizzling explained properly" (section "Results": swizzling the input
 * tiles against swizzling only the output tile), on gemm_run's own 256x256
 * kernel (8 waves, 16x16x32 MFMAs) for bf16 K-major A and B and a 16-bit D,
 * which that kernel stages in LDS (with a 16-bit C brought in by its last
 * loads).  operand_swz: 16 = the library's operand layout (16-byte units
 * XORed with the 256-byte bank-line index), 0 = no swizzle.  output_swz: 1 =
 * the C and D staging areas use their XOR keys (the library), 0 = logical
 * chunk order.  Every combination gives the same D bit for bit; only LDS
 * bank conflicts and speed differ.  The other arguments are gemm_run's, with
 * C NULL or 16-bit and d_dtype SG_BF16 or SG_F16.  Errors: as gemm_run, and
 * SG_ERR_SHAPE for another operand_swz or output_swz, SG_ERR_DTYPE for a
 * 32-bit C or D.
 */
int gemm_layout_io_run(int operand_swz, int output_swz, int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, const void* C, int c_dtype, void* D,
                       int d_dtype, void* stream);

/*
 * gemm_layout128_run -- gemm_layout_run on 128x128 tiles of the 4-wave
 * kernel (the 32x32x16 MFMA), where a padded layout also fits in LDS: the
 * padding alternative to swizzling weighed in "Swizzling explained properly"
 * (sections "Why swizzle?" and "Results").
 *   layout  16, 8 or 0 as gemm_layout_run's swz_units, or SG_LAYOUT_PAD16:
 *           no XOR, each 128-byte LDS row followed by 16 bytes of padding
 *           (loaded through registers, since padded rows do not tile the
 *           direct-to-LDS path's 1 KiB regions).
 * Every layout gives the same D.  Errors: as gemm_layout_run, SG_ERR_SHAPE
 * for another layout value.
 */
#define SG_LAYOUT_PAD16 (-1)
int gemm_layout128_run(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                       const void* B, const void* C, int c_dtype, void* D, int d_dtype,
                       void* stream);

/* Thread-local text of the last failing call ("" if none).  Never NULL. */
const char* gemm_last_error(void);

/* Library version and build description.  Never NULL. */
const char* gemm_version(void);

/*
 * gemm_lds_layout -- the LDS byte map the kernels use for a K-major operand
 * tile (host-side, no GPU needed).  Writes out[r * (row_bytes/16) + c] = the
 * byte offset within one LDS stage of logical 16-byte chunk c of tile row r,
 * for r < rows.  row_bytes is 64, 128 or 256; rows a positive multiple of 8.
 * The map is the XOR swizzle of "Swizzling explained properly" applied to
 * (bank line, 16-byte unit within the line), never splitting a 16-byte atom.
 * Returns SG_OK, SG_ERR_NULL or SG_ERR_SHAPE.
 */
int gemm_lds_layout(int rows, int row_bytes, int32_t* out);

/*
 * gemm_lds_layout_mxfp6 -- the LDS byte map of mxfp6_gemm_run's operand
 * tiles (host-side, no GPU needed).  Writes out[r * 12 + q] = the byte
 * offset within one LDS stage of bytes [8q, 8q + 8) of the 96 bytes of tile
 * row r, for r < rows.  The map is gemm_lds_layout's XOR swizzle for
 * 128-byte rows with every odd row displaced by 8 bytes, except the rows at
 * block position `unshifted` (row % 32 == unshifted; 32 for none), which the
 * kernel uses for the tile holding the operand's last row.  The displacement
 * lets 8-byte reads of 32 rows, which the XOR of 16-byte units alone maps
 * to 16 bank slots, reach all 32 ("Swizzling explained properly", section
 * "Why swizzle?": the bank arithmetic).  rows is a positive multiple of 32.
 * Returns SG_OK, SG_ERR_NULL or SG_ERR_SHAPE.
 */
int gemm_lds_layout_mxfp6(int rows, int unshifted, int32_t* out);

/*
 * gemm_lds_layout_cblock -- where the 256x256 bf16/fp16 kernel keeps a
 * 16-bit C in LDS for its epilogue (host-side, no GPU needed).  That kernel
 * reads C (the "+C" of the GEMM) through the loads of its last two K tiles,
 * which would otherwise fetch zeros past K, into the four half-tile ring
 * slots those loads fill.  Writes out[(w * 128 + r) * 8 + c], for wave
 * w < 4 of a 128-row group, row r < 128 and 16-byte chunk c < 8 of that
 * wave's 128 x 64 block of C: quarter r / 32 (which slot) times 16384 plus
 * the byte offset inside the slot's 16 KiB half.  The placement is an XOR
 * of the chunk index with a row key, the same construction as the operand
 * swizzle ("Swizzling explained properly", section "What does swizzling
 * do?"), chosen for 8-byte epilogue reads.  Returns SG_OK or SG_ERR_NULL.
 */
int gemm_lds_layout_cblock(int32_t* out);

/*
 * gemm_lds_image -- runs the kernels' global->LDS loader once for one operand
 * tile and copies the LDS stage out byte for byte, unswizzled by nothing.
 *   X         device operand, K-major [rows_total][K] of elem_bytes-sized
 *             elements (2 for f16/bf16, 1 for e4m3).
 *   tile_rows 128 or 256; the tile covers rows [row0, row0 + tile_rows)
 *             and the 128-byte K slice starting at element k0 (k0 * elem_bytes
 *             a multiple of 128).  Rows >= rows_total and k >= K read as zero.
 *   out       device buffer of tile_rows * 128 bytes.
 * Returns SG_OK or an SG_ERR_* code.
 */
int gemm_lds_image(const void* X, int64_t rows_total, int64_t K, int elem_bytes,
                   int64_t row0, int64_t k0, int tile_rows, void* out,
                   void* stream);

/*
 * Measurement support (not part of any GEMM call).
 *
 * gemm_clock_trace -- turns the clock trace of this thread's later launches
 * on (buf non-NULL) or off (buf NULL).  While on, every kernel of a gemm_run,
 * gemm_strided_run, gemm_layout_run, gemm_layout128_run, grouped_gemm_run,
 * mx_gemm_run, mxfp4_gemm_run or mxfp6_gemm_run call records, for each
 * workgroup b < slots, buf[4b .. 4b+3] = {shader-clock counter at its start,
 * the same at the end of its first wave, real-time counter at the start, the
 * same at the end}.  The shader-clock counter (s_memtime) advances once per
 * core clock; the real-time counter (s_memrealtime) at the constant rate
 * written to *wall_khz (kHz, the device attribute; NULL skips it).  So
 * (t_end - t_start) / (rt_end - rt_start) * wall_khz is the clock in kHz
 * that workgroup ran at: the clock the GEMM itself held, which sets its
 * clock-adjusted MFMA peak.  buf: DEVICE memory of 4 * slots uint64_t,
 * 8-byte aligned, alive while the trace is on.  The kernels only test the
 * pointer when the trace is off.  Errors: SG_ERR_SHAPE (slots < 0),
 * SG_ERR_ALIGN, SG_ERR_HIP.
 */
int gemm_clock_trace(void* buf, int64_t slots, int* wall_khz);

/*
 * gemm_clock_probe -- a kernel of W = gemm_clock_probe_waves() waves, one
 * workgroup of eight waves per CU of 256 CUs (two waves per SIMD, as the
 * 256x256 GEMM runs), each issuing `iters` rounds of 8 independent
 * v_mfma_f32_16x16x32_bf16 (16 cycles each) on random bf16 register
 * operands.  Wave w writes out[4w .. 4w+3] = {shader-clock counter at the
 * start of its loop, at the end, real-time counter at the start, at the end}
 * and out[4W + w] = bits of its fp32 accumulator sum.  Over a CU's eight
 * waves, 16 * 2 * 8 * iters cycles (the MFMAs of one SIMD) per real-time
 * span is the clock under a full MFMA load, and the shader-clock span over
 * the same real-time span shows whether the counter counts core clocks.
 * out: DEVICE memory of 5 * W uint64_t.  iters in [1, 2^24].  Errors:
 * SG_ERR_NULL, SG_ERR_ALIGN, SG_ERR_SHAPE, SG_ERR_HIP.
 */
int gemm_clock_probe(int64_t iters, void* out, void* stream);
int gemm_clock_probe_waves(void);

/*
 * gemm_last_kernel -- the kernel instantiation the last call on this thread
 * that launched one enqueued, as "name<parameters>" (for example
 * "pingpong16_gemm_kernel<bf16,k,k,swz16>"); "" before any launch.  Calls
 * that launch nothing (an error, an empty problem) leave it unchanged.
 * Thread-local; never NULL.
 */
const char* gemm_last_kernel(void);

/*
 * gemm_lds_image_tile -- runs one loader of the 256x256 kernels once, as the
 * first group of four waves of a workgroup issues it, and copies the LDS it
 * filled to `out` byte for byte, so that tests can hold the loaded image
 * against the byte map the fragment reads use ("Swizzling explained
 * properly", section "Sample swizzled matmul": the stores into the swizzled
 * tile and the reads out of it must use one map).
 *   X        DEVICE rows of `row_bytes` bytes (a multiple of 16), `rows` of
 *            them, 16-byte aligned; bytes past a row or rows past `rows`
 *            read as zero where the loader zero-fills.
 *   kind     SG_IMG_HALF / SG_IMG_HALF_KEXACT: a K-major 16-bit operand; the
 *              half tile of rows [row0, row0 + 128) and bytes [byte0, byte0
 *              + 128) (byte0 % 128 == 0) through the loader that checks K
 *              per load / the K-exact loader (row_bytes % 128 == 0).  The
 *              image is 16384 bytes laid out by gemm_lds_layout(128, 128).
 *            SG_IMG_MN256: an MN-major 16-bit operand [K = rows][row_bytes/2];
 *              k rows [row0, row0 + 64) (row0 % 64 == 0), columns [byte0/2,
 *              byte0/2 + 128) (byte0 % 256 == 0).  16384 bytes: byte b of
 *              k row r at 256 r + 32 ((b / 32) XOR key(r)) + b mod 32,
 *              key(r) = (r mod 4) + 4 (bit 3 of r).
 *            SG_IMG_FP6: an MXFP6 operand (row_bytes = 3K/4, a multiple of
 *              96); rows [row0, row0 + 128) of the 256-row tile at row0
 *              (row0 % 256 == 0), the K tile of bytes [byte0, byte0 + 96)
 *              (byte0 % 96 == 0).  16384 bytes laid out by
 *              gemm_lds_layout_mxfp6(128, u) with u the block position of
 *              the operand's last row if that row lies in this 256-row tile,
 *              else 32.
 *            SG_IMG_CBLOCK: a 16-bit C [rows][row_bytes/2]; the first 128
 *              rows of the 256 x 256 output tile at (row0, byte0/2) (row0 %
 *              256 == 0, byte0 % 512 == 0).  65536 bytes: the four
 *              quarters of gemm_lds_layout_cblock(), quarter Q at 16384 Q.
 *   out      DEVICE buffer of 16384 (65536 for SG_IMG_CBLOCK) bytes.
 * Errors: SG_ERR_NULL, SG_ERR_ALIGN, SG_ERR_SHAPE (origin not on the grid,
 * or outside the operand), SG_ERR_DTYPE (unknown kind), SG_ERR_HIP.
 */
#define SG_IMG_HALF 1
#define SG_IMG_HALF_KEXACT 2
#define SG_IMG_MN256 3
#define SG_IMG_FP6 4
#define SG_IMG_CBLOCK 5
int gemm_lds_image_tile(int kind, const void* X, int64_t rows, int64_t row_bytes,
                        int64_t row0, int64_t byte0, void* out, void* stream);

/*
 * gemm_mfma_scale_probe -- one v_mfma_scale_f32_32x32x64_f8f6f4 of one wave
 * with the format code fmt for both operands (0 e4m3, 2 e2m3, 3 e3m2, 4
 * e2m1), accumulating from zero: lane l (0..63) passes a[32 l .. 32 l + 31]
 * as its first source operand, b[32 l ..] as its second, and scale bytes
 * sa[l], sb[l] (byte 0 of each scale register).  out[16 l + r] receives
 * accumulator register r of lane l.  It exposes the scaled MFMA's operand
 * and scale layout -- which K element and which 32-element block each lane
 * and byte feed ("06 Blackwell Tensor Core - tcgen05 MMA", section
 * "Block-Scaled MMA", defines that placement for its own hardware) -- to
 * tests with one-hot operands.  a, b: DEVICE, 2048 bytes each; sa, sb: 64
 * bytes each; out: 4096 bytes (fp32).
 * Errors: SG_ERR_NULL, SG_ERR_ALIGN (a, b, out not 16-byte aligned),
 * SG_ERR_DTYPE (fmt), SG_ERR_HIP.
 */
int gemm_mfma_scale_probe(int fmt, const void* a, const void* b, const void* sa,
                          const void* sb, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIZZLED_GEMM_H */
