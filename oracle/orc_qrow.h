/*
 * orc_qrow.h -- declarations of the CPU oracle (test infrastructure only).
 *
 * The oracle is a plain, slow, single-threaded C implementation of
 * importance-matrix-weighted row quantization. It exists to check the GPU
 * library. Only the test-suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load it; the GPU library never does, and the two share
 * no code, headers or tables. Every constant below is the oracle's own copy.
 *
 * Floating-point contract: compiled with -ffp-contract=off and without
 * -ffast-math, so every float operation is one IEEE-754 binary32 operation
 * rounded to nearest-even, and fused multiply-adds appear only where fmaf()
 * is written.
 */
#ifndef ORC_QROW_H
#define ORC_QROW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Output formats (values fixed; the GPU library's enum must match). */
enum {
    ORC_Q4_0 = 0,    /* 32 weights, levels -8..7, fp32 scale              20 B */
    ORC_Q4_1 = 1,    /* 32 weights, levels 0..15, fp32 scale + fp32 min   24 B */
    ORC_Q5_0 = 2,    /* 32 weights, levels -16..15, fp32 scale            24 B */
    ORC_Q5_1 = 3,    /* 32 weights, levels 0..31, fp32 scale + fp32 min   28 B */
    ORC_Q4_K = 4,    /* 256 weights, 8x32 sub-blocks, 6-bit sc/mn, fp16 d 144 B */
    ORC_Q8_K128 = 5, /* 128 activations, fp32 d, int8, int16 sums/32     140 B */
    ORC_Q6_0 = 6,    /* 32 weights, levels -32..31, fp32 scale, 2-bit plane 28 B */
    ORC_Q8_K64 = 7,  /* 64 activations, fp32 d, int8, int16 sums/32       72 B */
    ORC_Q8_K16 = 8,  /* 16 activations, fp32 d, int8, int16 sum, 2 B pad   24 B */
    ORC_Q6_K = 9,    /* 256 weights, 16x16 sub-blocks, int8 sc, fp16 d, levels -32..31 212 B */
    ORC_Q5_K = 10    /* 256 weights, 8x32 sub-blocks, 6-bit sc/mn, fp16 d, levels 0..31 176 B */
};

/* Solver constants (the oracle's own copy). */
#define ORC_CAND_STEP       0.25f /* spacing of the trial scales, in levels   */
#ifndef ORC_SYM_CAND
#define ORC_SYM_CAND        5     /* trial scales, symmetric blocks           */
#endif
#ifndef ORC_SYM_FLIP_PASSES
#define ORC_SYM_FLIP_PASSES 1     /* greedy flip passes, symmetric blocks     */
#endif
#ifndef ORC_ASYM_CAND
#define ORC_ASYM_CAND       3     /* trial scales, asymmetric blocks          */
#endif
#ifndef ORC_ASYM_FLIP_PASSES
#define ORC_ASYM_FLIP_PASSES 1    /* greedy flip passes, asymmetric blocks    */
#endif

/* Return codes. */
#define ORC_OK       0
#define ORC_EINVAL  -1

/* Fills c[0..5] = {step*4 (as int), sym cand, sym passes, asym cand,
 * asym passes, max block length}; lets a test compare the two copies. */
void orc_solver_constants(int32_t *c);

size_t orc_block_bytes(int type);
int    orc_block_elems(int type);
size_t orc_row_bytes(int type, int64_t n_per_row);   /* 0 if invalid */

/* Row statistic: sigma2 = (sum of x^2 in double) / n, rounded once to float.
 * orc_row_sigma2_f64 returns the value before that last rounding. */
float  orc_row_sigma2(const float *x, int64_t n);
double orc_row_sigma2_f64(const float *x, int64_t n);

/* Element importances w_j = q_j * sqrtf(fmaf(x_j, x_j, sigma2)); q == NULL
 * means q_j = 1. */
void orc_row_weights(const float *x, const float *q, int64_t n, float sigma2,
                     float *w);

/* Weightings: w_j = q_j * m(x_j) with m one of the magnitude forms below
 * (values fixed; the GPU library's enum must match). */
enum {
    ORC_W_SQRT_SIGMA2_X2 = 0,   /* sqrtf(fmaf(x, x, sigma2)) -- the default */
    ORC_W_X2 = 1,               /* x * x                                     */
    ORC_W_ABS_X = 2,            /* |x|                                       */
    ORC_W_SIGMA2_PLUS_X2 = 3,   /* fmaf(x, x, sigma2)                        */
    ORC_W_SIGMA_PLUS_ABS_X = 4, /* sqrtf(sigma2) + |x|                       */
    ORC_W_IMATRIX_ONLY = 5      /* 1                                          */
};
void orc_row_weights_mode(const float *x, const float *q, int64_t n,
                          float sigma2, int mode, float *w);
/* orc_quantize_rows with a weighting; with a group of all-zero importances
 * the same weighting is taken with q = 1. */
int orc_quantize_rows_weighted(int type, const float *x, const float *imatrix,
                               int64_t n_rows, int64_t n_per_row, int mode,
                               uint8_t *out);
int orc_quantize_row_sigma2_mode(int type, const float *x, const float *q,
                                 int64_t n_per_row, float sigma2, int mode,
                                 uint8_t *out);

/* Block solvers on n <= 256 elements with explicit weights w.
 * info[0] = index of the winning trial scale (-1: zero block),
 * info[1] = flips accepted, info[2] = passes run,
 * info[3] = 1 if the last pass run accepted nothing (converged).
 * Symmetric: levels l in [-nmax, nmax-1] returned in l_out (signed).
 * Asymmetric: levels in [0, nmax]; k4 != 0 selects the Q4_K sub-block rules
 * (range widened to include 0, offset m <= 0). */
int orc_solve_sym(int n, const float *x, const float *w, int nmax, int K, int F,
                  int8_t *l_out, float *d_out, int32_t *info);
int orc_solve_asym(int n, const float *x, const float *w, int nmax, int K,
                   int F, int k4, uint8_t *l_out, float *d_out, float *m_out,
                   int32_t *info);

/* Weight-row quantizers: x is [n_rows, n_per_row] fp32 row-major; imatrix
 * is [n_per_row] (or NULL); out holds n_rows * orc_row_bytes() bytes. */
int orc_quantize_rows(int type, const float *x, const float *imatrix,
                      int64_t n_rows, int64_t n_per_row, uint8_t *out);
/* Grouped: imatrix is [n_groups, n_per_row]; row r uses group r / rpg. */
int orc_quantize_rows_grouped(int type, const float *x, const float *imatrix,
                              int64_t n_groups, int64_t rows_per_group,
                              int64_t n_per_row, uint8_t *out);
/* One row with the row statistic supplied by the caller. */
int orc_quantize_row_sigma2(int type, const float *x, const float *q,
                            int64_t n_per_row, float sigma2, uint8_t *out);

/* How the Q4_K 6-bit sub-scales and sub-offsets are chosen (other types
 * have none and ignore it). */
enum {
    ORC_FIT_MAX = 0,       /* fp16(max/63), each rounded to the nearest level */
    ORC_FIT_WEIGHTED = 1   /* weighted least-squares fit of the eight values   */
};
/* Weighted fit v_j ~ d * l_j, l_j in 0..nmax, of n values v_j >= 0 with
 * weights W_j: K trial scales, F flip passes (the sub-scale fit). */
int orc_fit_levels_pos(int n, const float *v, const float *W, int nmax, int K,
                       int F, uint8_t *l_out, float *d_out, int32_t *info);
/* One row with the row statistic supplied, a weighting and a sub-scale fit. */
int orc_quantize_row_sigma2_ex(int type, const float *x, const float *q,
                               int64_t n_per_row, float sigma2, int mode,
                               int fit, uint8_t *out);
/* Grouped rows with a weighting and a sub-scale fit. */
int orc_quantize_rows_ex(int type, const float *x, const float *imatrix,
                         int64_t n_groups, int64_t rows_per_group,
                         int64_t n_per_row, int mode, int fit, uint8_t *out);

/* Q8_K_128 activation quantizer. */
int orc_quantize_q8k128(const float *x, int64_t n_rows, int64_t n_per_row,
                        uint8_t *out);
/* The Q8_K family by block size: type is ORC_Q8_K128, ORC_Q8_K64 or
 * ORC_Q8_K16. */
int orc_quantize_q8k(int type, const float *x, int64_t n_rows,
                     int64_t n_per_row, uint8_t *out);

/* Decoder for every format above. */
int orc_dequantize_rows(int type, const uint8_t *in, int64_t n_rows,
                        int64_t n_per_row, float *out);

/* Importance-matrix accumulator (imatrix_oracle.c). State: sums
 * [n_experts, n_cols] double and counts [n_experts], added to in place.
 * act is [n_tokens, n_slots, n_cols]; ids is [n_tokens, top_k] or NULL for
 * a dense tensor (then n_experts == 1 and n_slots == 1). */
int orc_imatrix_accumulate(const float *act, int64_t n_tokens, int64_t n_slots,
                           int64_t n_cols, const int32_t *ids, int64_t top_k,
                           int64_t n_experts, double *sums, int64_t *counts);
int orc_imatrix_merge(double *sums, int64_t *counts, const double *src_sums,
                      const int64_t *src_counts, int64_t n_experts,
                      int64_t n_cols);
/* q = sums / count in double, rounded once to float; 0 where count == 0. */
int orc_imatrix_finalize(const double *sums, const int64_t *counts,
                         int64_t n_experts, int64_t n_cols, float *q);

/* Product of quantized weight rows w [n_out, row_bytes(type, n_in)] with
 * Q8_K_128 activation rows x [n_tok, row_bytes(Q8_K128, n_in)] (matmul_oracle.c):
 * y[t * n_out + r] = sum_i w[r][i] * a[t][i] in double over the exact decoded
 * values; s_abs (or NULL) receives sum_i (|scale part| + |offset part|)*|a_i|. */
int orc_matmul_q8k128(int type, const uint8_t *w, const uint8_t *x,
                      int64_t n_out, int64_t n_tok, int64_t n_in, double *y,
                      double *s_abs);
/* The same product with activations of any Q8_K block size (act_type
 * ORC_Q8_K128, ORC_Q8_K64 or ORC_Q8_K16). */
int orc_matmul_q8k(int type, int act_type, const uint8_t *w, const uint8_t *x,
                   int64_t n_out, int64_t n_tok, int64_t n_in, double *y,
                   double *s_abs);
/* The same product for Q4_1/Q5_1 weights with fp32 activations quantized to
 * Q8_1 (32 values, fp16 d and fp16 s = d * sum(q)), the offset part taken
 * from s, in float: the formulation whose s overflows. */
int orc_matmul_q8_1(int type, const uint8_t *w, const float *x, int64_t n_out,
                    int64_t n_tok, int64_t n_in, float *y);

/* Error statistics of packed rows against the rows they came from
 * (stats_oracle.c): sums[7] = {sum e^2, sum x^2, sum q e^2, sum q x^2,
 * RMSE, relative RMSE, importance-weighted relative RMSE} in double,
 * e = x - xhat in float; *max_abs = max |e|; *p95_abs = the ceil(0.95 N)-th
 * smallest |e|. q (or NULL) is per column. */
int orc_quantize_stats(int type, const float *x, const uint8_t *packed,
                       const float *q, int64_t n_rows, int64_t n_per_row,
                       double *sums, float *max_abs, float *p95_abs);

/* IEEE-754 binary16 conversions (round to nearest-even, subnormals kept). */
uint16_t orc_f32_to_f16(float f);
float    orc_f16_to_f32(uint16_t h);

#ifdef __cplusplus
}
#endif
#endif
