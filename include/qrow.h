/*
 * qrow.h -- C-ABI of libqrow.so: importance-matrix-weighted row quantization
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
 *       的由来与原理", section 一: per row, sigma2 is the mean of x^2; each element
 *       gets the importance w = qw * sqrt(sigma2 + x^2), qw being the imatrix
 *       (diagonal Hessian estimate) entry of its column; each block's scale is
 *       the weighted least-squares value sumlx/suml2, refined by greedy level
 *       flips along g = scale*w*(x - scale*l).
 *  [KQ] "3.2 K-quants 与重要性矩阵：量化兵器谱", section 一: the Q4_K super-block
 *       (fp16 super-scale over 6-bit sub-scales); Q5_K_M among the K types.
 *  [LQ] "从零理解 LLM 量化 PTQ、QAT 与 ik_llama.cpp 量化体系的源码级导学",
 *       section 2.1: the legacy 32-weight blocks Q4_0, Q4_1, Q5_0, Q5_1;
 *       section 2.2: the K-quant family, Q5_K among it.
 *  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …", section 修复方案:
 *       the Q8_K_128 activation block; the row length must be a multiple of
 *       128.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are caller-owned DEVICE pointers (HIP device memory or
 *    managed memory visible to the current device), 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL: the default stream). Every call only
 *    enqueues work on that stream and returns; the caller synchronizes.
 *  - The library allocates no device memory and keeps no state between
 *    calls, except the thread-local error string.
 *  - Rows are stored contiguously (row-major, no padding); the packed output
 *    of a row is qr_row_bytes(type, n_per_row) bytes and row r starts at
 *    byte r * qr_row_bytes(type, n_per_row).
 *  - Return value 0 on success, a negative QR_E* code on failure. On failure
 *    nothing is launched and qr_last_error() describes the problem.
 *  - n_rows == 0 is a successful no-op.
 *  - Inputs must be finite. Importances must be finite and >= 0 (they are
 *    sums of squared activations); this is not checked on the device.
 *
 * Packed block layouts (little-endian; the pages give bit widths, these byte
 * layouts are this library's):
 *  Q4_0  20 B: f32 d | u8 qs[16]            levels l in -8..7,  code u = l+8
 *  Q4_1  24 B: f32 d | f32 m | u8 qs[16]    levels 0..15,       x ~ d*u + m
 *  Q5_0  24 B: f32 d | u32 qh | u8 qs[16]   levels -16..15,     u = l+16
 *  Q5_1  28 B: f32 d | f32 m | u32 qh | u8 qs[16]   levels 0..31
 *     qs[i] holds u_i (low nibble) and u_{i+16} (high nibble); bit i of qh
 *     is bit 4 of u_i.
 *  Q6_0  28 B: f32 d | u8 qh[8] | u8 qs[16]  levels -32..31,     u = l+32
 *     qs as above holds the low 4 bits; bits 2i and 2i+1 of the 64-bit
 *     little-endian qh are bits 4 and 5 of u_i.
 *  Q6_K 212 B per 256: f16 d | 2 zero bytes | i8 s[16] | qs[8][16] | qh[8][8]
 *     16 sub-blocks of 16 weights, levels -32..31 (u = l+32) decoding to
 *     (f32(d)*s_j)*(u - 32); 32-weight group g uses qs[g] (nibbles as above:
 *     the low nibbles are sub-block 2g, the high ones 2g+1) and the 2-bit
 *     plane qh[g] as in Q6_0.
 *  Q4_K 144 B per 256: f16 d | f16 dmin | sc[8] as 6-bit fields in 6 B |
 *     mn[8] as 6-bit fields in 6 B | u8 qs[128]; field j sits at bit 6j;
 *     sub-block j (32 weights) uses qs[16j .. 16j+15] as above and decodes
 *     to (d*sc_j)*u - dmin*mn_j.
 *  Q5_K 176 B per 256: the Q4_K header (16 B) | qh[8] as u32 | u8 qs[128];
 *     levels 0..31: sub-block j takes bit 4 of u_i from bit i of qh[j] and
 *     the low 4 bits from qs[16j .. 16j+15] (nibbles as above); decodes as
 *     Q4_K. (The pages name Q5_K but give no layout: it is Q4_K's
 *     super-block with one more bit per weight, 5.5 bits per weight.)
 *  Q8_K128 140 B per 128: f32 d | i8 q[128] | i16 bsum[4]; bsum[g] is the
 *     plain sum of q[32g .. 32g+31], not multiplied by d.
 *  Q8_K64   72 B per 64:  f32 d | i8 q[64] | i16 bsum[2] (sums of 32 codes).
 *  Q8_K16   24 B per 16:  f32 d | i8 q[16] | i16 bsum | 2 zero bytes.
 */
#ifndef QROW_H
#define QROW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QR_Q4_0 = 0,
    QR_Q4_1 = 1,
    QR_Q5_0 = 2,
    QR_Q5_1 = 3,
    QR_Q4_K = 4,
    QR_Q8_K128 = 5,
    QR_Q6_0 = 6,
    QR_Q8_K64 = 7,
    QR_Q8_K16 = 8,
    QR_Q6_K = 9,
    QR_Q5_K = 10
} qr_type;

typedef enum { QR_F32 = 0, QR_BF16 = 1 } qr_dtype;

/* Element importance w = q * m(x) [WT 一, 二]: the pages' form and the
 * magnitude forms the pages list as tried before it, for ablation. */
typedef enum {
    QR_W_SQRT_SIGMA2_X2 = 0,    /* m = sqrtf(fmaf(x, x, sigma2))  (the pages') */
    QR_W_X2 = 1,                /* m = x * x                                   */
    QR_W_ABS_X = 2,             /* m = |x|                                     */
    QR_W_SIGMA2_PLUS_X2 = 3,    /* m = fmaf(x, x, sigma2)                      */
    QR_W_SIGMA_PLUS_ABS_X = 4,  /* m = sqrtf(sigma2) + |x|                     */
    QR_W_IMATRIX_ONLY = 5       /* m = 1: the imatrix alone                    */
} qr_weighting;

#define QR_OK            0
#define QR_EINVAL_TYPE  -1  /* unknown type, or a type the call does not take */
#define QR_EINVAL_SHAPE -2  /* n_per_row not a positive multiple of the block
                               length (32, 256 or 128), above the supported
                               maximum, a negative count, or more rows than
                               one launch holds (row quantizers: see below)  */
#define QR_EINVAL_PTR   -3  /* NULL or misaligned pointer with n_rows > 0    */
#define QR_EOVERFLOW    -4  /* a size computation overflows                  */
#define QR_EDEVICE      -5  /* the HIP runtime reported an error            */

/* Largest supported row: the row is staged in LDS while its blocks are
 * solved (32-value groups padded to 144 bytes for fp32 and 80 for bf16, plus
 * the cross-wave partial sums, within the 160 KiB of one workgroup). */
#define QR_MAX_ROW_F32   32768
#define QR_MAX_ROW_BF16  32768

/*
 * qr_quantize_rows -- importance-weighted quantization of weight rows [WT 一],
 * [KQ 一], [LQ 2.1].
 *  t        QR_Q4_0, QR_Q4_1, QR_Q5_0, QR_Q5_1, QR_Q6_0, QR_Q4_K, QR_Q5_K or
 *           QR_Q6_K (else EINVAL_TYPE).
 *  src      QR_F32 or QR_BF16: element type of x.
 *  x        [n_rows, n_per_row] weights, row-major.
 *  imatrix  [n_per_row] fp32 importances shared by all rows, or NULL for
 *           unit importances.
 *  out      n_rows * qr_row_bytes(t, n_per_row) bytes, written completely.
 * Per row: sigma2 = (sum x^2, accumulated in double) / n_per_row rounded to
 * float; w_j = imatrix[j] * sqrtf(fmaf(x_j, x_j, sigma2)); a 32-weight group
 * whose w are all zero uses imatrix = 1 instead. Each 32-weight block (Q4_K:
 * sub-block) is fitted by a trial-scale search, the weighted least-squares
 * scale (and offset), and greedy flip passes; Q4_K (levels 0..15) and Q5_K
 * (0..31) then quantize the eight sub-scales and offsets to 6 bits under
 * fp16 super-scales and re-round the levels. Q6_K fits each 16-weight sub-block with the symmetric routine on
 * levels -32..31, sets d = fp16(max |d_j| / 127) and s_j = rint(d_j / d)
 * in -127..127, and re-rounds the levels against d*s_j ([KQ 一]'s two-level
 * scaling at 6 bits; the layout is this library's). The results are
 * bit-identical to the CPU oracle of this project.
 * Row limit: each row is one workgroup of 64 * min(8, ceil(n_per_row / 2048))
 * threads, and one launch holds fewer than 2^32 threads, so n_rows must be
 * at most (2^32 - 1) / that thread count (67108863 rows of 2048 values,
 * 8388607 rows of 16384 or more); larger calls return QR_EINVAL_SHAPE
 * before anything is launched (split them). This applies to every row
 * quantizer below (for the grouped forms, to n_groups * rows_per_group).
 */
int qr_quantize_rows(int t, int src, const void *x, const float *imatrix,
                     int64_t n_rows, int64_t n_per_row, void *out,
                     void *stream);

/*
 * qr_quantize_rows_grouped -- as qr_quantize_rows for a stack of matrices
 * that share a shape but not an imatrix (e.g. the experts of an MoE layer),
 * in one launch. x is [n_groups * rows_per_group, n_per_row]; imatrix is
 * [n_groups, n_per_row] (or NULL); row r uses imatrix row r / rows_per_group.
 */
int qr_quantize_rows_grouped(int t, int src, const void *x,
                             const float *imatrix, int64_t n_groups,
                             int64_t rows_per_group, int64_t n_per_row,
                             void *out, void *stream);

/*
 * qr_quantize_rows_weighted -- qr_quantize_rows with another element
 * importance: w_j = imatrix[j] * m(x_j) with m given by `weighting`
 * (qr_weighting; QR_EINVAL_TYPE otherwise). A 32-weight group whose w are
 * all zero uses imatrix = 1 with the same m. QR_W_SQRT_SIGMA2_X2 gives
 * exactly the output of qr_quantize_rows. The results are bit-identical to
 * the CPU oracle of this project for every weighting.
 */
int qr_quantize_rows_weighted(int t, int src, const void *x,
                              const float *imatrix, int64_t n_rows,
                              int64_t n_per_row, int weighting, void *out,
                              void *stream);

/* How the Q4_K and Q5_K 6-bit sub-scales and sub-offsets are chosen (types
 * without them ignore it). */
typedef enum {
    QR_FIT_MAX = 0,       /* d = fp16(max a_j / 63), sc_j = rint(a_j / d): the default */
    QR_FIT_WEIGHTED = 1   /* weighted least-squares fit of the eight values */
} qr_subscale_fit;

/*
 * qr_quantize_rows_ex -- the row quantizer with every option: grouped
 * importances (as qr_quantize_rows_grouped), a weighting (as
 * qr_quantize_rows_weighted) and the Q4_K/Q5_K sub-scale fit. [KQ 一] fixes eight
 * 6-bit sub-scales and sub-offsets under fp16 super-scales but not how they
 * are chosen. With QR_FIT_WEIGHTED the sub-blocks' least-squares scales a_j
 * (and offsets b_j) are fitted as a_j ~ d * sc_j, sc_j in 0..63, by the
 * weighted least squares with trial scales and greedy flips of [WT 一],
 * each sub-block weighted by the sum of its 32 importances: trial scales
 * put the largest value on 63 + 0.25k (k = 0, -1, +1, -2, +2), levels are
 * rounded in float, the sums, comparisons and flips are evaluated in double
 * and d = sumlx/suml2 is stored as fp16 (sub-scales 0 if that is 0). The
 * element codes are then re-rounded against the stored scales as in the
 * default. Errors as qr_quantize_rows_grouped, and QR_EINVAL_TYPE for an
 * unknown weighting or subscale_fit. The default choices (QR_W_SQRT_SIGMA2_X2,
 * QR_FIT_MAX) give the bytes of qr_quantize_rows_grouped.
 */
int qr_quantize_rows_ex(int t, int src, const void *x, const float *imatrix,
                        int64_t n_groups, int64_t rows_per_group,
                        int64_t n_per_row, int weighting, int subscale_fit,
                        void *out, void *stream);

/*
 * qr_quantize_activations_q8k128 -- the Q8_K_128 activation quantizer
 * [Q8 修复方案]. Per 128 values: amax = max |x|; codes q = rint(x * (127/amax))
 * in -127..127; d = amax / 127 stored as f32; bsum[g] = sum of 32 codes as
 * int16, not multiplied by d. An all-zero block (or one whose 127/amax is
 * not finite) stores d = 0 and zero codes. n_per_row must be a multiple of
 * 128. x is fp32 or bf16 [n_rows, n_per_row]; out holds
 * n_rows * qr_row_bytes(QR_Q8_K128, n_per_row) bytes.
 */
int qr_quantize_activations_q8k128(int src, const void *x, int64_t n_rows,
                                   int64_t n_per_row, void *out, void *stream);

/*
 * qr_quantize_activations_q8k -- the Q8_K activation family by block size
 * [Q8 修复方案 for the 128-value block; 技术启示与后续演进 names Q8_K64 and
 * Q8_K16 as later members built on the same idea: an f32 scale and integer
 * code sums that are not multiplied by it]. t is QR_Q8_K128, QR_Q8_K64 or
 * QR_Q8_K16; each block of B = 128, 64 or 16 values is quantized exactly as
 * above (amax, rint(x * 127/amax), d = amax/127) and stored as
 *   Q8_K64: [f32 d][i8 q[64]][i16 bsum[2]]              72 bytes
 *   Q8_K16: [f32 d][i8 q[16]][i16 bsum][2 zero bytes]   24 bytes
 * with bsum the sum of each 32 codes (of the block's 16 codes for Q8_K16),
 * little-endian. n_per_row must be a positive multiple of B; out holds
 * n_rows * qr_row_bytes(t, n_per_row) bytes. Errors as above, and
 * QR_EINVAL_TYPE for any other t.
 */
int qr_quantize_activations_q8k(int t, int src, const void *x, int64_t n_rows,
                                int64_t n_per_row, void *out, void *stream);

/*
 * qr_dequantize_rows -- decoder for every type above. in is the packed
 * [n_rows, qr_row_bytes(t, n_per_row)] buffer; out is fp32
 * [n_rows, n_per_row]. Symmetric blocks decode to d*(u - nmax), asymmetric
 * ones to fmaf(d, u, m), Q4_K and Q5_K to fmaf(f32(d)*sc, u, -(f32(dmin)*mn)), the
 * Q8_K family to d*q.
 */
int qr_dequantize_rows(int t, const void *in, int64_t n_rows,
                       int64_t n_per_row, float *out, void *stream);

/* Packed bytes of one row; 0 if t is unknown or n_per_row is not a
 * non-negative multiple of the block length. */
size_t qr_row_bytes(int t, int64_t n_per_row);

/* Elements per block: 32, 256, 128, 64 or 16; 0 for an unknown type. */
int qr_block_elems(int t);

/* Fills c[0..5] = {4 * trial-scale step, symmetric trials, symmetric flip
 * passes, asymmetric trials, asymmetric flip passes, 32}: the solver
 * constants compiled into the library. */
void qr_solver_constants(int32_t *c);

/* Message for the last failing call on this thread ("" if none). Valid
 * until the next call on the same thread. */
const char *qr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
