/*
 * tgemm_ref.c -- CPU oracle for C = ReLU(A @ B) on binary16 inputs.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never links it and
 * shares no code, header, table or helper with it.
 *
 * What it computes (the plain definition, written out):
 *   "Writing high-performance kernels in TileLang, from GEMM to MLA" (atlascloud.ai),
 *   section "Let's write a GEMM": the kernel computes C = ReLU(A @ B) with A (M x K),
 *   B (K x N), C (M x N), all float16, a float accumulator cleared before the K loop,
 *   an elementwise max(C, 0) after it, and a write-back to float16.
 *   "TileLang-MUSA operator development" (7yue.com), section 3 (first kernel: GEMM):
 *   the same contraction without the ReLU, float32 accumulator, checked against A @ B
 *   computed in float32.
 *
 * Reading taken here: every input is first decoded exactly from its binary16 bits to
 * double; the sum over k runs in ascending k in double. A product of two binary16
 * values has at most 22 significant bits, so each product is exact in double and the
 * only roundings are the K-1 double additions, in a fixed order. The result is
 * returned in double, before any rounding to binary16. ReLU is x > 0 ? x : +0.0 (the
 * page's max(x, 0); -0 and NaN map to +0).
 *
 * Row-major, element (i, j) of X at X[i * ldX + j]. No blocking, no reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0: value = (-1)^s * f * 2^-24 (zero and subnormals)
 * exponent 1..30: value = (-1)^s * (1024 + f) * 2^(e - 25)
 * exponent 31: infinity (f = 0) or NaN (f != 0). */
double oracle_f16_decode(uint16_t h) {
    int s = h >> 15;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e < 31)
        v = ldexp((double)(1024 + f), e - 25);
    else
        v = f ? NAN : INFINITY;
    return s ? -v : v;
}

/* Decode n binary16 values to double. */
void oracle_f16_decode_array(const uint16_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f16_decode(src[i]);
}

/* Round a double to the nearest binary16, ties to even; |x| >= 65520 goes to +-inf
 * (65520 is the midpoint between the largest finite value 65504 and 2^16, and the tie
 * goes to the even significand, which is the overflow). NaN -> 0x7E00 with the sign. */
uint16_t oracle_f16_encode_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7E00;
    double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1): floor(log2 a) = e2 - 1 */
    int ex = e2 - 1;
    if (ex < -14) ex = -14; /* below the normal range the spacing stays 2^-24 */
    /* Spacing of binary16 values in [2^ex, 2^(ex+1)) is 2^(ex-10); n < 2048 exactly. */
    double n = ldexp(a, 10 - ex);
    double r = nearbyint(n); /* default rounding mode: to nearest, ties to even */
    int64_t q = (int64_t)r;
    if (q >= 2048) { q >>= 1; ex += 1; } /* rounding carried into the next binade */
    if (q < 1024) return sign | (uint16_t)q; /* subnormal (ex == -14 only) */
    int biased = ex + 15;
    if (biased >= 31) return sign | 0x7C00;
    return sign | (uint16_t)((biased << 10) | (int)(q - 1024));
}

void oracle_f16_encode_array(const double* src, uint16_t* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f16_encode_rne(src[i]);
}

static double relu_d(double x) { return x > 0.0 ? x : 0.0; }

/* Full product: C[i*ldc + j] = relu?( sum_{k ascending} A[i,k] * B[k,j] ), in double.
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 if the decode buffer for B
 * cannot be allocated. */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda,
                    const uint16_t* B, int64_t ldb,
                    double* C, int64_t ldc, int relu, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc(sizeof(double) * (size_t)K * (size_t)N);
        if (!Bd) return -1;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j) Bd[k * N + j] = oracle_f16_decode(B[k * ldb + j]);
    }
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i) {
        double* acc = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_f16_decode(A[i * lda + k]);
            const double* brow = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j) acc[j] = relu_d(acc[j]);
    }
    free(Bd);
    return 0;
}

/* Selected entries, one at a time: out[t] = relu?( sum_k A[rows[t],k] * B[k,cols[t]] ),
 * k ascending -- the same additions in the same order as oracle_gemm_f16, so the two
 * agree bit for bit. For large shapes where the whole product is too slow. */
void oracle_gemm_f16_entries(int64_t K,
                             const uint16_t* A, int64_t lda,
                             const uint16_t* B, int64_t ldb,
                             int64_t count, const int64_t* rows, const int64_t* cols,
                             double* out, int relu, int nthreads) {
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
    for (int64_t t = 0; t < count; ++t) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_f16_decode(A[rows[t] * lda + k]) * oracle_f16_decode(B[k * ldb + cols[t]]);
        out[t] = relu ? relu_d(acc) : acc;
    }
}

/* Threads the OpenMP runtime would use by default (reported with timings). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
