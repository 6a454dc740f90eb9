/*
 * gemm_oracle.c -- plain, slow, CPU reference for the swizzled GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header or table
 * with the HIP kernels.
 *
 * What it computes (fp64 accumulation over exactly decoded inputs):
 *
 *   dense   ref[i][j]   = sum_k a(i,k) * b(k,j) + c(i,j)
 *           bound[i][j] = sum_k |a(i,k) * b(k,j)| + |c(i,j)|
 *     The tensor-core operation D = A*B + C ("Tensor Cores, layouts, and
 *     swizzling", opening section; "Swizzling explained properly", sample
 *     swizzled matmul).  With a NULL C the "enable-input-d = false" form
 *     D = A*B is computed ("06 Blackwell Tensor Core - tcgen05 MMA", operand
 *     table).  a(i,k) = A[i*K+k] when A is K-major, A[k*M+i] when MN-major;
 *     b(k,j) = B[j*K+k] when B is K-major, B[k*N+j] when MN-major.
 *
 *   mx      ref[i][j] = sum_blk 2^(SFA[i][blk]-127) * 2^(SFB[j][blk]-127)
 *                        * sum_{k in blk} e4m3(A[i][k]) * e4m3(B[j][k])
 *     Block-scaled MMA: output (m,n) uses scale SFA[m,sfk] for A and
 *     SFB[n,sfk] for B ("06 Blackwell Tensor Core", Block-Scaled MMA).  The
 *     32-element K block and the e8m0 scale type are not on that page; they
 *     are the MXFP8 workload's definition.  MXFP4 is the same sum over e2m1
 *     elements (two per byte, element 2i in the low nibble of byte i);
 *     MXFP6 over OCP e2m3 or e3m2 elements stored as a 6-bit stream per
 *     row (element k at bits [6k, 6k+6), little endian).
 *
 * Products of two 16-bit floats (and of two e4m3) are exact in fp64; the
 * fp64 sum of K terms is within (K-1)*2^-53 * bound of the exact value.
 *
 * Every entry point returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F16 = 1, ORC_BF16 = 2, ORC_F32 = 3, ORC_E4M3 = 4, ORC_E8M0 = 5, ORC_E2M1 = 6,
       ORC_E2M3 = 7, ORC_E3M2 = 8 };
enum { ORC_K_MAJOR = 0, ORC_MN_MAJOR = 1 };

/* ---------------------------------------------------------------- decode */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);             /* subnormal: m * 2^-14 / 2^10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32. */
static double dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double dec_f32(const void *p) {
    float f;
    memcpy(&f, p, 4);
    return (double)f;
}

/* OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinity,
 * S.1111.111 is NaN; the largest finite magnitude is 448. */
static double dec_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 fraction bit; no infinity
 * or NaN; the largest magnitude is 6. */
static double dec_e2m1(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v;
    if (e == 0)
        v = 0.5 * m;                           /* m/2 * 2^(1-1) */
    else
        v = ldexp((double)(2 + m), e - 2);     /* (1 + m/2) * 2^(e-1) */
    return s ? -v : v;
}

/* OCP FP6 E2M3: 1 sign, 2 exponent (bias 1), 3 fraction bits; no infinity
 * or NaN; the largest magnitude is 7.5. */
static double dec_e2m3(uint8_t c) {
    int s = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
    double v;
    if (e == 0)
        v = ldexp((double)m, -3);              /* m/8 * 2^(1-1) */
    else
        v = ldexp((double)(8 + m), e - 4);     /* (1 + m/8) * 2^(e-1) */
    return s ? -v : v;
}

/* OCP FP6 E3M2: 1 sign, 3 exponent (bias 3), 2 fraction bits; no infinity
 * or NaN; the largest magnitude is 28. */
static double dec_e3m2(uint8_t c) {
    int s = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
    double v;
    if (e == 0)
        v = ldexp((double)m, -4);              /* m/4 * 2^(1-3) */
    else
        v = ldexp((double)(4 + m), e - 5);     /* (1 + m/4) * 2^(e-3) */
    return s ? -v : v;
}

/* Element idx of a packed 6-bit stream: bits [6 idx, 6 idx + 6), little
 * endian (bit 0 of the stream is bit 0 of byte 0). */
static uint8_t code6_at(const uint8_t *p, int64_t idx) {
    int64_t bit = 6 * idx;
    int64_t byte = bit >> 3;
    int sh = (int)(bit & 7);
    unsigned w = p[byte];
    if (sh > 2) w |= (unsigned)p[byte + 1] << 8;
    return (uint8_t)((w >> sh) & 63);
}

/* OCP E8M0 scale: 2^(e-127); 0xFF is NaN. */
static double dec_e8m0(uint8_t b) {
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
}

static int elem_size(int dt) {
    switch (dt) {
    case ORC_F16: case ORC_BF16: return 2;
    case ORC_F32: return 4;
    case ORC_E4M3: case ORC_E8M0: return 1;
    case ORC_E2M1: return 1;  /* two elements per byte; indices count elements */
    case ORC_E2M3: case ORC_E3M2: return 1;  /* four elements per three bytes */
    default: return 0;
    }
}

static double dec_at(int dt, const void *base, int64_t idx) {
    const uint8_t *p = (const uint8_t *)base;
    switch (dt) {
    case ORC_F16: { uint16_t h; memcpy(&h, p + 2 * idx, 2); return dec_f16(h); }
    case ORC_BF16: { uint16_t h; memcpy(&h, p + 2 * idx, 2); return dec_bf16(h); }
    case ORC_F32: return dec_f32(p + 4 * idx);
    case ORC_E4M3: return dec_e4m3(p[idx]);
    case ORC_E8M0: return dec_e8m0(p[idx]);
    case ORC_E2M1: return dec_e2m1((idx & 1) ? (uint8_t)(p[idx >> 1] >> 4) : (uint8_t)(p[idx >> 1] & 15));
    case ORC_E2M3: return dec_e2m3(code6_at(p, idx));
    case ORC_E3M2: return dec_e3m2(code6_at(p, idx));
    default: return NAN;
    }
}

/* Decode n elements of dtype dt into fp64. */
int oracle_decode(int dt, const void *src, int64_t n, double *dst) {
    if (!src || !dst || n < 0 || elem_size(dt) == 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = dec_at(dt, src, i);
    return 0;
}

/* ------------------------------------------------------------- threading */

typedef struct {
    void (*fn)(void *ctx, int64_t row_begin, int64_t row_end);
    void *ctx;
    int64_t rows;
    int nthreads;
    int tid;
} worker_t;

static void *worker_main(void *arg) {
    worker_t *w = (worker_t *)arg;
    int64_t per = (w->rows + w->nthreads - 1) / w->nthreads;
    int64_t b = per * w->tid, e = b + per;
    if (e > w->rows) e = w->rows;
    if (b < e) w->fn(w->ctx, b, e);
    return NULL;
}

/* Runs fn over [0, rows) split into contiguous row ranges, one per thread.
 * nthreads <= 0 means every online host core. */
static void parallel_rows(void (*fn)(void *, int64_t, int64_t), void *ctx,
                          int64_t rows, int nthreads) {
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    if (nthreads <= 1) {
        fn(ctx, 0, rows);
        return;
    }
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    worker_t *ws = (worker_t *)calloc((size_t)nthreads, sizeof(worker_t));
    for (int t = 0; t < nthreads; ++t) {
        ws[t] = (worker_t){fn, ctx, rows, nthreads, t};
        pthread_create(&th[t], NULL, worker_main, &ws[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(ws);
}

int oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ----------------------------------------------------------------- dense */

typedef struct {
    int64_t M, N, K;
    const double *a;   /* [M][K] decoded, K contiguous */
    const double *b;   /* [N][K] decoded, K contiguous */
    double alpha, beta;
    const void *C;     /* element (i, j) at C[i * ldc + j]; NULL: no C */
    int64_t ldc;
    int c_dtype;
    double *ref, *bound;
} dense_ctx;

static void dense_rows(void *vctx, int64_t i0, int64_t i1) {
    const dense_ctx *x = (const dense_ctx *)vctx;
    for (int64_t i = i0; i < i1; ++i) {
        const double *ai = x->a + i * x->K;
        for (int64_t j = 0; j < x->N; ++j) {
            const double *bj = x->b + j * x->K;
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < x->K; ++k) {
                double p = ai[k] * bj[k];
                s += p;
                sa += fabs(p);
            }
            double c = x->C ? dec_at(x->c_dtype, x->C, i * x->ldc + j) : 0.0;
            x->ref[i * x->N + j] = x->alpha * s + x->beta * c;
            if (x->bound)
                x->bound[i * x->N + j] = fabs(x->alpha) * sa + fabs(x->beta) * fabs(c);
        }
    }
}

/* Logical row r (0..R-1) of an operand whose logical shape is R x K,
 * decoded to fp64 with K contiguous.  major == K: X[r*ld+k]; MN: X[k*ld+r]. */
static void expand_operand(int dt, const void *X, int major, int64_t R,
                           int64_t K, int64_t ld, double *out) {
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = dec_at(dt, X, major == ORC_K_MAJOR ? r * ld + k
                                                                : k * ld + r);
}

/* D = alpha * sum_k A(m,k) B(k,n) + beta * C(m,n) with leading dimensions in
 * elements: A(m,k) = A[m*lda+k] (K-major) or A[k*lda+m] (MN-major), B(k,n) =
 * B[n*ldb+k] or B[k*ldb+n], C(m,n) = C[m*ldc+n].  alpha == 0: A and B are not
 * read; beta == 0 or C == NULL: C is not read.  ref/bound are [M][N]
 * row-major fp64 (bound may be NULL): bound = |alpha| sum|a*b| + |beta| |c|. */
int oracle_gemm_ex(int64_t M, int64_t N, int64_t K, double alpha, const void *A,
                   int64_t lda, int a_major, const void *B, int64_t ldb, int b_major,
                   int ab_dtype, double beta, const void *C, int64_t ldc, int c_dtype,
                   double *ref, double *bound, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || !ref) return -1;
    if ((ab_dtype != ORC_F16 && ab_dtype != ORC_BF16) ||
        (a_major != ORC_K_MAJOR && a_major != ORC_MN_MAJOR) ||
        (b_major != ORC_K_MAJOR && b_major != ORC_MN_MAJOR))
        return -1;
    if (alpha == 0.0) K = 0;
    if (beta == 0.0) C = NULL;
    if (C && (elem_size(c_dtype) == 0 || ldc < N)) return -1;
    if (lda < (a_major == ORC_K_MAJOR ? K : M) || ldb < (b_major == ORC_K_MAJOR ? K : N))
        return -1;
    if (K > 0 && ((M > 0 && !A) || (N > 0 && !B))) return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!a || !b) { free(a); free(b); return -1; }
    if (K > 0) {
        expand_operand(ab_dtype, A, a_major, M, K, lda, a);
        expand_operand(ab_dtype, B, b_major, N, K, ldb, b);
    }
    dense_ctx x = {M, N, K, a, b, alpha, beta, C, ldc, c_dtype, ref, bound};
    parallel_rows(dense_rows, &x, M, nthreads);
    free(a);
    free(b);
    return 0;
}

/* D = A*B (+C) with packed operands: oracle_gemm_ex with alpha = beta = 1. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, const void *A, int a_major,
                const void *B, int b_major, int ab_dtype, const void *C,
                int c_dtype, double *ref, double *bound, int nthreads) {
    return oracle_gemm_ex(M, N, K, 1.0, A, a_major == ORC_K_MAJOR ? K : M, a_major, B,
                          b_major == ORC_K_MAJOR ? K : N, b_major, ab_dtype, 1.0, C, N,
                          c_dtype, ref, bound, nthreads);
}

/* The same definition evaluated only at the listed (row, col) points, each
 * straight from the stored operands; for outputs too large to form whole. */
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, const void *A,
                       int a_major, const void *B, int b_major, int ab_dtype,
                       const void *C, int c_dtype, int64_t npts,
                       const int64_t *rows, const int64_t *cols, double *ref,
                       double *bound) {
    if (M < 0 || N < 0 || K < 0 || npts < 0 || !ref || (npts && (!rows || !cols)))
        return -1;
    if ((ab_dtype != ORC_F16 && ab_dtype != ORC_BF16) ||
        (a_major != ORC_K_MAJOR && a_major != ORC_MN_MAJOR) ||
        (b_major != ORC_K_MAJOR && b_major != ORC_MN_MAJOR))
        return -1;
    for (int64_t p = 0; p < npts; ++p) {
        int64_t i = rows[p], j = cols[p];
        if (i < 0 || i >= M || j < 0 || j >= N) return -1;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double av = dec_at(ab_dtype, A, a_major == ORC_K_MAJOR ? i * K + k : k * M + i);
            double bv = dec_at(ab_dtype, B, b_major == ORC_K_MAJOR ? j * K + k : k * N + j);
            s += av * bv;
            sa += fabs(av * bv);
        }
        double c = C ? dec_at(c_dtype, C, i * N + j) : 0.0;
        ref[p] = s + c;
        if (bound) bound[p] = sa + fabs(c);
    }
    return 0;
}

/* -------------------------------------------------------------------- mx */

typedef struct {
    int64_t M, N, K, nblk;
    const double *a, *b;      /* decoded elements, [rows][K] */
    const double *sa, *sb;    /* decoded e8m0, [rows][K/32] */
    double *ref, *bound;
} mx_ctx;

static void mx_rows(void *vctx, int64_t i0, int64_t i1) {
    const mx_ctx *x = (const mx_ctx *)vctx;
    for (int64_t i = i0; i < i1; ++i) {
        for (int64_t j = 0; j < x->N; ++j) {
            double s = 0.0, sabs = 0.0;
            for (int64_t blk = 0; blk < x->nblk; ++blk) {
                const double *ai = x->a + i * x->K + blk * 32;
                const double *bj = x->b + j * x->K + blk * 32;
                double bs = 0.0, bsa = 0.0;
                for (int k = 0; k < 32; ++k) {
                    double p = ai[k] * bj[k];
                    bs += p;
                    bsa += fabs(p);
                }
                double scale = x->sa[i * x->nblk + blk] * x->sb[j * x->nblk + blk];
                s += scale * bs;
                sabs += scale * bsa;
            }
            x->ref[i * x->N + j] = s;
            if (x->bound) x->bound[i * x->N + j] = sabs;
        }
    }
}

/* A [M][K], SFA e8m0 [M][K/32], B [N][K], SFB e8m0 [N][K/32]; the elements
 * are e4m3 (fmt ORC_E4M3, one per byte), e2m1 (ORC_E2M1, two per byte) or
 * e2m3 / e3m2 (ORC_E2M3 / ORC_E3M2, a 6-bit stream: four per three bytes). */
int oracle_mx_gemm_fmt(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                       const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB,
                       double *ref, double *bound, int nthreads) {
    if (fmt != ORC_E4M3 && fmt != ORC_E2M1 && fmt != ORC_E2M3 && fmt != ORC_E3M2) return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || !ref) return -1;
    if (K > 0 && ((M > 0 && (!A || !SFA)) || (N > 0 && (!B || !SFB)))) return -1;
    int64_t nblk = K / 32;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    double *sa = (double *)malloc(sizeof(double) * (size_t)(M * nblk + 1));
    double *sb = (double *)malloc(sizeof(double) * (size_t)(N * nblk + 1));
    if (!a || !b || !sa || !sb) { free(a); free(b); free(sa); free(sb); return -1; }
    if (K > 0) {
        oracle_decode(fmt, A, M * K, a);
        oracle_decode(fmt, B, N * K, b);
        oracle_decode(ORC_E8M0, SFA, M * nblk, sa);
        oracle_decode(ORC_E8M0, SFB, N * nblk, sb);
    }
    mx_ctx x = {M, N, K, nblk, a, b, sa, sb, ref, bound};
    parallel_rows(mx_rows, &x, M, nthreads);
    free(a); free(b); free(sa); free(sb);
    return 0;
}

int oracle_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *A,
                   const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB,
                   double *ref, double *bound, int nthreads) {
    return oracle_mx_gemm_fmt(ORC_E4M3, M, N, K, A, SFA, B, SFB, ref, bound, nthreads);
}

int oracle_mx_gemm_points_fmt(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                              const uint8_t *SFA, const uint8_t *B,
                              const uint8_t *SFB, int64_t npts,
                              const int64_t *rows, const int64_t *cols,
                              double *ref, double *bound) {
    if (fmt != ORC_E4M3 && fmt != ORC_E2M1 && fmt != ORC_E2M3 && fmt != ORC_E3M2) return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || npts < 0 || !ref ||
        (npts && (!rows || !cols)))
        return -1;
    int64_t nblk = K / 32;
    for (int64_t p = 0; p < npts; ++p) {
        int64_t i = rows[p], j = cols[p];
        if (i < 0 || i >= M || j < 0 || j >= N) return -1;
        double s = 0.0, sabs = 0.0;
        for (int64_t blk = 0; blk < nblk; ++blk) {
            double bs = 0.0, bsa = 0.0;
            for (int k = 0; k < 32; ++k) {
                double pr = dec_at(fmt, A, i * K + blk * 32 + k) *
                            dec_at(fmt, B, j * K + blk * 32 + k);
                bs += pr;
                bsa += fabs(pr);
            }
            double scale = dec_e8m0(SFA[i * nblk + blk]) * dec_e8m0(SFB[j * nblk + blk]);
            s += scale * bs;
            sabs += scale * bsa;
        }
        ref[p] = s;
        if (bound) bound[p] = sabs;
    }
    return 0;
}

int oracle_mx_gemm_points(int64_t M, int64_t N, int64_t K, const uint8_t *A,
                          const uint8_t *SFA, const uint8_t *B,
                          const uint8_t *SFB, int64_t npts,
                          const int64_t *rows, const int64_t *cols,
                          double *ref, double *bound) {
    return oracle_mx_gemm_points_fmt(ORC_E4M3, M, N, K, A, SFA, B, SFB, npts, rows, cols,
                                     ref, bound);
}
