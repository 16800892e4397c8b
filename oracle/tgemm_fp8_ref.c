/*
 * tgemm_fp8_ref.c -- CPU oracle for the fp8 block-scaled GEMM and its block quantizer.
 *
 * TEST INFRASTRUCTURE ONLY, like tgemm_ref.c (built into the same library): only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it; the GPU
 * library shares no code, header, table or helper with it.
 *
 * What the pages fix and what is read into them:
 *   "TileLang-MUSA operator development" (7yue.com), section 8.2 (reusing TileKernels)
 *   calls fp8_block_scaled_linear(x, w_fp8, scale_w, block=128): a linear layer whose
 *   weight is stored in fp8 with one scale per block of 128; the TileLang write-up measured
 *   on A100 (nxmr.cn 138173), section 7, names the scaling strategy: per-block scales as in
 *   CUTLASS. Nothing on the pages fixes the fp8 encoding, the block shapes, the scale type
 *   or how x is brought to fp8. The reading taken here (the block-scaled recipe those
 *   names refer to):
 *     - fp8 = OCP E4M3 ("E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 fraction bits, no
 *       infinities, S.1111.111 = NaN, largest finite 448;
 *     - x (M x K, activations) is quantized per 1 x 128 block (one row, 128 consecutive
 *       k), the weight W (N x K) per 128 x 128 block; scales are float32, one per block,
 *       and a block's real values are code * scale;
 *     - Y = X_q W_q^T with the scales applied per 128-wide k-block:
 *         C[i,j] = relu?( sum_kb  SA[i,kb] * SB[j/128,kb] * sum_{k in kb} a[i,k] * w[j,k] )
 *       where a, w are the decoded codes; C is returned unrounded (double);
 *     - the quantizer of a block with largest magnitude amax (float32):
 *         s = amax / 448 (float32 division; s = 1 for an all-zero block),
 *         q = e4m3(x / s) (float32 division, then round to nearest even, saturating to
 *         +-448; NaN -> NaN code). Inputs are finite binary16 values.
 *
 * Exactness: an E4M3 value is an integer multiple of 2^-9 below 2^9, so a product of two
 * is a multiple of 2^-18 below 2^18, and a sum of at most 128 such products is a multiple
 * of 2^-18 below 2^25: it needs at most 43 significant bits and is exact in double. The
 * product SA * SB of two float32 values is exact in double as well. The only roundings
 * are one multiplication per block and the additions over blocks (kb ascending).
 *
 * Row-major, element (i, j) of X at X[i * ldX + j]; SA is M x KB and SB is
 * ceil(N/128) x KB, both row-major and contiguous, KB = ceil(K/128).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double oracle_f16_decode(uint16_t h); /* tgemm_ref.c */

#define FP8_BLOCK 128

/* E4M3: exponent field 0 -> (-1)^s * f * 2^-9 (zero and subnormals);
 * 1..15 -> (-1)^s * (8 + f) * 2^(e - 10), except e = 15, f = 7 which is NaN. */
double oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7;
    int e = (c >> 3) & 15;
    int f = c & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8 + f), e - 10);
    return s ? -v : v;
}

void oracle_e4m3_decode_array(const uint8_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_e4m3_decode(src[i]);
}

/* Nearest E4M3 value, ties to the even fraction, magnitudes at or above 448 saturate to
 * 448 (the rounding could only go to 480, which is the NaN pattern), NaN -> 0x7F with the
 * sign. Below 2^-6 the spacing stays 2^-9 (subnormals). */
uint8_t oracle_e4m3_encode_sat(double x) {
    uint8_t sign = signbit(x) ? 0x80 : 0;
    if (isnan(x)) return sign | 0x7F;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int ex = e2 - 1;
    if (ex < -6) ex = -6;   /* subnormal range: spacing 2^-9 = 2^(-6-3) */
    double n = ldexp(a, 3 - ex); /* in units of the spacing 2^(ex-3); n < 16 */
    int64_t q = (int64_t)nearbyint(n);
    if (q >= 16) { q >>= 1; ex += 1; } /* carried into the next binade */
    if (q < 8) return sign | (uint8_t)q; /* subnormal: only when ex == -6 */
    int biased = ex + 7;
    return sign | (uint8_t)((biased << 3) | (int)(q - 8)); /* a < 448 keeps this finite */
}

void oracle_e4m3_encode_array(const double* src, uint8_t* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_e4m3_encode_sat(src[i]);
}

/* Block quantizer: X (R x K binary16, ldx) -> Q (R x K E4M3 codes, ldq) and S
 * (ceil(R/block_rows) x KB float32, contiguous), blocks of block_rows x 128. */
void oracle_quant_fp8(int64_t R, int64_t K, const uint16_t* X, int64_t ldx, int64_t block_rows,
                      uint8_t* Q, int64_t ldq, float* S) {
    const int64_t KB = (K + FP8_BLOCK - 1) / FP8_BLOCK;
    const int64_t RB = (R + block_rows - 1) / block_rows;
    for (int64_t rb = 0; rb < RB; ++rb) {
        const int64_t r0 = rb * block_rows, r1 = r0 + block_rows < R ? r0 + block_rows : R;
        for (int64_t kb = 0; kb < KB; ++kb) {
            const int64_t k0 = kb * FP8_BLOCK, k1 = k0 + FP8_BLOCK < K ? k0 + FP8_BLOCK : K;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t k = k0; k < k1; ++k) {
                    const float v = (float)fabs(oracle_f16_decode(X[r * ldx + k]));
                    if (v > amax) amax = v;
                }
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            S[rb * KB + kb] = s;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t k = k0; k < k1; ++k) {
                    const float y = (float)oracle_f16_decode(X[r * ldx + k]) / s;
                    Q[r * ldq + k] = oracle_e4m3_encode_sat((double)y);
                }
        }
    }
}

static double relu_d(double x) { return x > 0.0 ? x : 0.0; }

/* One output element: the definition above, blocks ascending, k ascending inside. */
static double fp8_entry(int64_t K, int64_t KB, const uint8_t* arow, const float* sarow,
                        const uint8_t* wrow, const float* sbrow) {
    double acc = 0.0;
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int64_t k0 = kb * FP8_BLOCK, k1 = k0 + FP8_BLOCK < K ? k0 + FP8_BLOCK : K;
        double p = 0.0; /* exact */
        for (int64_t k = k0; k < k1; ++k) p += oracle_e4m3_decode(arow[k]) * oracle_e4m3_decode(wrow[k]);
        acc += ((double)sarow[kb] * (double)sbrow[kb]) * p;
    }
    return acc;
}

/* Full product. A: M x K codes (lda), B: N x K codes (ldb), SA: M x KB, SB: ceil(N/128)
 * x KB, C: M x N doubles (ldc). */
int oracle_gemm_fp8_block(int64_t M, int64_t N, int64_t K,
                          const uint8_t* A, int64_t lda, const float* SA,
                          const uint8_t* B, int64_t ldb, const float* SB,
                          double* C, int64_t ldc, int relu, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
    const int64_t KB = (K + FP8_BLOCK - 1) / FP8_BLOCK;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            const double v = fp8_entry(K, KB, A + i * lda, SA + i * KB, B + j * ldb, SB + (j / FP8_BLOCK) * KB);
            C[i * ldc + j] = relu ? relu_d(v) : v;
        }
    return 0;
}

/* Selected entries (rows[t], cols[t]), bitwise equal to oracle_gemm_fp8_block. */
void oracle_gemm_fp8_block_entries(int64_t K, const uint8_t* A, int64_t lda, const float* SA,
                                   const uint8_t* B, int64_t ldb, const float* SB,
                                   int64_t count, const int64_t* rows, const int64_t* cols,
                                   double* out, int relu, int nthreads) {
    const int64_t KB = (K + FP8_BLOCK - 1) / FP8_BLOCK;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        const double v = fp8_entry(K, KB, A + i * lda, SA + i * KB, B + j * ldb, SB + (j / FP8_BLOCK) * KB);
        out[t] = relu ? relu_d(v) : v;
    }
}

/* Per-element magnitude bound used by the tolerance of the fp8 path:
 *   E[i,j] = sum_kb |SA[i,kb] * SB[j/128,kb]| * max_{k in kb}|a[i,k]| * max_{k in kb}|w[j,k]|
 * (an upper bound of sum_kb |scale| * max_k |a w|, the size of the largest term of each
 * block), for the full M x N matrix into out (row-major, N per row). */
void oracle_fp8_block_bound(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                            const float* SA, const uint8_t* B, int64_t ldb, const float* SB,
                            double* out) {
    const int64_t KB = (K + FP8_BLOCK - 1) / FP8_BLOCK;
    double* am = (double*)malloc(sizeof(double) * (size_t)(M * KB + 1));
    double* bm = (double*)malloc(sizeof(double) * (size_t)(N * KB + 1));
    if (!am || !bm) { free(am); free(bm); return; }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t kb = 0; kb < KB; ++kb) {
            double m = 0.0;
            for (int64_t k = kb * FP8_BLOCK; k < K && k < (kb + 1) * FP8_BLOCK; ++k)
                m = fmax(m, fabs(oracle_e4m3_decode(A[i * lda + k])));
            am[i * KB + kb] = m * fabs((double)SA[i * KB + kb]);
        }
    for (int64_t j = 0; j < N; ++j)
        for (int64_t kb = 0; kb < KB; ++kb) {
            double m = 0.0;
            for (int64_t k = kb * FP8_BLOCK; k < K && k < (kb + 1) * FP8_BLOCK; ++k)
                m = fmax(m, fabs(oracle_e4m3_decode(B[j * ldb + k])));
            bm[j * KB + kb] = m * fabs((double)SB[(j / FP8_BLOCK) * KB + kb]);
        }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double e = 0.0;
            for (int64_t kb = 0; kb < KB; ++kb) e += am[i * KB + kb] * bm[j * KB + kb];
            out[i * N + j] = e;
        }
    free(am);
    free(bm);
}
