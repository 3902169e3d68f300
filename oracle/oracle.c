/*
 * CPU oracle for the GEMM + bias + ReLU hot path and for the LDS-staged copy.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load this file or
 * the library built from it: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg call it. It shares no code, header or constant
 * with the GPU library.
 *
 * Sources (the three web pages on warp specialization):
 *   [KP]  pwwt.cn/news/4436243, the Chinese article on intra-kernel
 *         pipelining with TMA and mbarrier, section 4.1: float A[M,K] and
 *         B[K,N], output C[M,N] = A*B + bias passed through a ReLU.
 *   [WS]  aicassindra.com, "GPU warp specialization", section "End-to-end
 *         flow": an output tile accumulates the products of many K-dimension
 *         tiles of A and B.
 *   [PC]  willy-chan.github.io, "Producer-Consumer Warp Specialization for
 *         TMA Operations": the staged copy moves data into a shared-memory
 *         buffer and out to global memory unchanged.
 *
 * Readings where the pages are silent:
 *   - bias has one entry per output column n and is added once, after the
 *     full K sum, then the ReLU is applied;
 *   - relu(s) = s for s > 0, NaN stays NaN, everything else (including -0)
 *     becomes +0;
 *   - layouts are dense row-major: A[m*K+k], B[k*N+n], C[m*N+n];
 *   - K = 0 is an empty sum (C = relu(bias)); M = 0 or N = 0 writes nothing.
 *
 * Precision: every product of two fp32 (or bf16) values is exact in fp64,
 * so the only rounding is the fp64 additions, done in ascending k order for
 * every element. The loops below are blocked over rows and columns only; the
 * k order of each element's sum is never changed.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_RB 16  /* rows of C per block */
#define ORACLE_JB 512 /* columns of C per block */

static double relu64(double s) {
    if (s > 0.0) return s;
    if (s != s) return s; /* NaN propagates */
    return 0.0;           /* +0 for zero, -0 and negatives */
}

static double bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * C[m][n] = relu( sum_{k ascending} A[m][k] * B[k][n] + bias[n] ), all fp64.
 * A is M x K, B is K x N, bias has N entries, C is M x N (fp64, row-major).
 */
static void gemm_core(int64_t M, int64_t N, int64_t K, const double *A,
                      const double *B, const double *bias, double *C) {
    int64_t nrb = (M + ORACLE_RB - 1) / ORACLE_RB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rb = 0; rb < nrb; ++rb) {
        int64_t i0 = rb * ORACLE_RB;
        int64_t i1 = i0 + ORACLE_RB < M ? i0 + ORACLE_RB : M;
        for (int64_t j0 = 0; j0 < N; j0 += ORACLE_JB) {
            int64_t j1 = j0 + ORACLE_JB < N ? j0 + ORACLE_JB : N;
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j) C[i * N + j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double *brow = B + k * N;
                for (int64_t i = i0; i < i1; ++i) {
                    double a = A[i * K + k];
                    double *crow = C + i * N;
                    for (int64_t j = j0; j < j1; ++j) crow[j] += a * brow[j];
                }
            }
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j)
                    C[i * N + j] = relu64(C[i * N + j] + bias[j]);
        }
    }
}

/* Widen an fp32 (dtype 0) or bf16-bits (dtype 1) array to fp64. */
static double *widen(int dtype, const void *src, int64_t n) {
    double *d = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!d) return NULL;
    if (dtype == 0) {
        const float *s = (const float *)src;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) d[i] = (double)s[i];
    } else {
        const uint16_t *s = (const uint16_t *)src;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) d[i] = bf16_to_f64(s[i]);
    }
    return d;
}

/*
 * Full GEMM + bias + ReLU. dtype 0: A, B, bias are float; dtype 1: they are
 * bf16 bit patterns (uint16), widened exactly. Returns 0, or -1 on bad
 * arguments, -2 when host memory runs out.
 */
int oracle_gemm_bias_relu(int dtype, int64_t M, int64_t N, int64_t K,
                          const void *A, const void *B, const void *bias,
                          double *C, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || (dtype != 0 && dtype != 1)) return -1;
    if (M == 0 || N == 0) return 0;
    set_threads(nthreads);
    double *Ad = widen(dtype, A, M * K);
    double *Bd = widen(dtype, B, K * N);
    double *bd = widen(dtype, bias, N);
    int rc = 0;
    if (!Ad || !Bd || !bd) rc = -2;
    else gemm_core(M, N, K, Ad, Bd, bd, C);
    free(Ad);
    free(Bd);
    free(bd);
    return rc;
}

/*
 * The same result for a chosen list of rows only: out is nrows x N, row r of
 * out is row rows[r] of C. Used to check very large products by sampling.
 */
int oracle_gemm_bias_relu_rows(int dtype, int64_t M, int64_t N, int64_t K,
                               const void *A, const void *B, const void *bias,
                               const int64_t *rows, int64_t nrows, double *out,
                               int nthreads) {
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || (dtype != 0 && dtype != 1)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;
    set_threads(nthreads);
    size_t esz = dtype == 0 ? sizeof(float) : sizeof(uint16_t);
    unsigned char *Asub = (unsigned char *)malloc((size_t)(nrows * K > 0 ? nrows * K : 1) * esz);
    if (!Asub) return -2;
    for (int64_t r = 0; r < nrows; ++r)
        memcpy(Asub + (size_t)(r * K) * esz, (const unsigned char *)A + (size_t)(rows[r] * K) * esz,
               (size_t)K * esz);
    int rc = oracle_gemm_bias_relu(dtype, nrows, N, K, Asub, B, bias, out, nthreads);
    free(Asub);
    return rc;
}

/*
 * Single elements, each as its own plain dot product in ascending k:
 * out[i] = C[ms[i]][ns[i]].
 */
int oracle_gemm_bias_relu_at(int dtype, int64_t M, int64_t N, int64_t K,
                             const void *A, const void *B, const void *bias,
                             const int64_t *ms, const int64_t *ns, int64_t count,
                             double *out, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || count < 0 || (dtype != 0 && dtype != 1)) return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double s = 0.0;
        if (dtype == 0) {
            const float *a = (const float *)A, *b = (const float *)B;
            for (int64_t k = 0; k < K; ++k) s += (double)a[m * K + k] * (double)b[k * N + n];
            s += (double)((const float *)bias)[n];
        } else {
            const uint16_t *a = (const uint16_t *)A, *b = (const uint16_t *)B;
            for (int64_t k = 0; k < K; ++k) s += bf16_to_f64(a[m * K + k]) * bf16_to_f64(b[k * N + n]);
            s += bf16_to_f64(((const uint16_t *)bias)[n]);
        }
        out[i] = relu64(s);
    }
    return 0;
}

/*
 * Staged-copy oracle: the result of the copy is the source, byte for byte.
 * Splits the range over threads; returns 0.
 */
int oracle_copy(const void *src, void *dst, uint64_t bytes, int nthreads) {
    set_threads(nthreads);
    const uint64_t chunk = 1u << 22;
    int64_t nchunks = (int64_t)((bytes + chunk - 1) / chunk);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nchunks; ++c) {
        uint64_t lo = (uint64_t)c * chunk;
        uint64_t n = bytes - lo < chunk ? bytes - lo : chunk;
        memcpy((unsigned char *)dst + lo, (const unsigned char *)src + lo, n);
    }
    return 0;
}

/* Index of the first differing byte of a and b over n bytes, or -1. */
int64_t oracle_first_mismatch(const void *a, const void *b, uint64_t n) {
    const unsigned char *x = (const unsigned char *)a, *y = (const unsigned char *)b;
    for (uint64_t i = 0; i < n; ++i)
        if (x[i] != y[i]) return (int64_t)i;
    return -1;
}

/* Number of OpenMP threads a parallel region would use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
