/*
 * oracle_driver.c -- runs every entry point of oracle/gemm_oracle.c on
 * small, exactly sized heap buffers, for an AddressSanitizer +
 * UndefinedBehaviorSanitizer build of the oracle (test infrastructure).
 * Checks a few results against a naive integer loop; any sanitizer report
 * aborts the run.  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode(int dt, const void *src, int64_t n, double *dst);
int oracle_default_threads(void);
int oracle_gemm(int64_t M, int64_t N, int64_t K, const void *A, int a_major, const void *B,
                int b_major, int ab_dtype, const void *C, int c_dtype, double *ref,
                double *bound, int nthreads);
int oracle_gemm_ex(int64_t M, int64_t N, int64_t K, double alpha, const void *A, int64_t lda,
                   int a_major, const void *B, int64_t ldb, int b_major, int ab_dtype,
                   double beta, const void *C, int64_t ldc, int c_dtype, double *ref,
                   double *bound, int nthreads);
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, const void *A, int a_major,
                       const void *B, int b_major, int ab_dtype, const void *C, int c_dtype,
                       int64_t n, const int64_t *rows, const int64_t *cols, double *ref,
                       double *bound);
int oracle_mx_gemm_fmt(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                       const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB, double *ref,
                       double *bound, int nthreads);
int oracle_mx_gemm_points_fmt(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                              const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB,
                              int64_t n, const int64_t *rows, const int64_t *cols,
                              double *ref, double *bound);

static int fails = 0;
#define EXPECT(c)                                                        \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
                    __LINE__, #c);                                       \
            ++fails;                                                     \
        }                                                                \
    } while (0)

/* bf16 bits of a small integer (exact). */
static uint16_t bf16_of(int v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

int main(void) {
    const int64_t M = 7, N = 12, K = 24;
    int threads[2] = {1, 3};

    /* decode: every code of every element type */
    for (int dt = 1; dt <= 8; ++dt) {
        int64_t n = dt == 3 ? 64 : (dt == 1 || dt == 2) ? 65536 : 256;
        size_t bytes = dt == 3 ? 256 : (dt == 1 || dt == 2) ? 131072 : 256;
        uint8_t *src = xmalloc(bytes);
        for (size_t i = 0; i < bytes; ++i) src[i] = (uint8_t)(i * 131u + (i >> 8));
        if (dt == 6) n = 512;            /* e2m1: two per byte */
        if (dt == 7 || dt == 8) n = 340; /* 6-bit stream: 255 bytes hold 340 */
        double *dst = xmalloc((size_t)n * sizeof(double));
        EXPECT(oracle_decode(dt, src, n, dst) == 0);
        free(src);
        free(dst);
    }

    /* dense, all majorness, integer values, against a naive loop */
    int a[7][24], b[12][24];
    for (int i = 0; i < M; ++i)
        for (int k = 0; k < K; ++k) a[i][k] = (i * 7 + k * 3) % 9 - 4;
    for (int j = 0; j < N; ++j)
        for (int k = 0; k < K; ++k) b[j][k] = (j * 5 + k) % 9 - 4;
    for (int am = 0; am < 2; ++am)
        for (int bm = 0; bm < 2; ++bm)
            for (int t = 0; t < 2; ++t) {
                uint16_t *A = xmalloc(M * K * 2), *B = xmalloc(N * K * 2);
                float *C = xmalloc(M * N * 4);
                for (int i = 0; i < M; ++i)
                    for (int k = 0; k < K; ++k)
                        A[am ? k * M + i : i * K + k] = bf16_of(a[i][k]);
                for (int j = 0; j < N; ++j)
                    for (int k = 0; k < K; ++k)
                        B[bm ? k * N + j : j * K + k] = bf16_of(b[j][k]);
                for (int i = 0; i < M * N; ++i) C[i] = (float)(i % 5);
                double *ref = xmalloc(M * N * 8), *bound = xmalloc(M * N * 8);
                EXPECT(oracle_gemm(M, N, K, A, am, B, bm, 2, C, 3, ref, bound, threads[t]) == 0);
                for (int i = 0; i < M; ++i)
                    for (int j = 0; j < N; ++j) {
                        long s = 0;
                        for (int k = 0; k < K; ++k) s += (long)a[i][k] * b[j][k];
                        EXPECT(ref[i * N + j] == (double)(s + (i * N + j) % 5));
                    }
                EXPECT(oracle_gemm(M, N, K, A, am, B, bm, 2, NULL, 0, ref, NULL, threads[t]) == 0);
                /* strided, padded rows, alpha and beta */
                int64_t lda = (am ? M : K) + 8, ldb = (bm ? N : K) + 4, ldc = N + 4;
                uint16_t *Ap = xmalloc((am ? K : M) * lda * 2), *Bp = xmalloc((bm ? K : N) * ldb * 2);
                float *Cp = xmalloc(M * ldc * 4);
                memset(Ap, 0, (am ? K : M) * lda * 2);
                memset(Bp, 0, (bm ? K : N) * ldb * 2);
                memset(Cp, 0, M * ldc * 4);
                EXPECT(oracle_gemm_ex(M, N, K, 2.0, Ap, lda, am, Bp, ldb, bm, 2, -3.0, Cp, ldc, 3,
                                      ref, bound, threads[t]) == 0);
                int64_t rows[3] = {0, 3, M - 1}, cols[3] = {N - 1, 0, 5};
                double pr[3], pb[3];
                EXPECT(oracle_gemm_points(M, N, K, A, am, B, bm, 2, C, 3, 3, rows, cols, pr, pb) == 0);
                free(A); free(B); free(C); free(ref); free(bound); free(Ap); free(Bp); free(Cp);
            }
    /* bad arguments */
    {
        double r[4];
        EXPECT(oracle_gemm(-1, 2, 2, NULL, 0, NULL, 0, 2, NULL, 0, r, NULL, 1) != 0);
        EXPECT(oracle_gemm(2, 2, 2, NULL, 7, NULL, 0, 2, NULL, 0, r, NULL, 1) != 0);
    }

    /* block-scaled, every element format; K = 128 (4 scale blocks) */
    const int fmts[4] = {4, 6, 7, 8};
    for (int f = 0; f < 4; ++f) {
        const int64_t MK = 5, NK = 9, KK = 128;
        int64_t rb = fmts[f] == 4 ? KK : fmts[f] == 6 ? KK / 2 : KK * 3 / 4;
        uint8_t *A = xmalloc(MK * rb), *B = xmalloc(NK * rb);
        uint8_t *SA = xmalloc(MK * KK / 32), *SB = xmalloc(NK * KK / 32);
        for (int64_t i = 0; i < MK * rb; ++i) A[i] = (uint8_t)((i * 37) & 0x7e);
        for (int64_t i = 0; i < NK * rb; ++i) B[i] = (uint8_t)((i * 53) & 0x7e);
        for (int64_t i = 0; i < MK * KK / 32; ++i) SA[i] = (uint8_t)(120 + i % 9);
        for (int64_t i = 0; i < NK * KK / 32; ++i) SB[i] = (uint8_t)(125 + i % 5);
        double *ref = xmalloc(MK * NK * 8), *bound = xmalloc(MK * NK * 8);
        for (int t = 0; t < 2; ++t)
            EXPECT(oracle_mx_gemm_fmt(fmts[f], MK, NK, KK, A, SA, B, SB, ref, bound, threads[t]) == 0);
        int64_t rows[2] = {0, MK - 1}, cols[2] = {NK - 1, 2};
        double pr[2], pb[2];
        EXPECT(oracle_mx_gemm_points_fmt(fmts[f], MK, NK, KK, A, SA, B, SB, 2, rows, cols, pr, pb) == 0);
        EXPECT(pr[0] == ref[NK - 1] && pr[1] == ref[(MK - 1) * NK + 2]);
        free(A); free(B); free(SA); free(SB); free(ref); free(bound);
    }
    EXPECT(oracle_default_threads() >= 1);
    if (fails) {
        fprintf(stderr, "%d expectation(s) failed\n", fails);
        return 1;
    }
    puts("oracle sanitizer run clean");
    return 0;
}
