/*
 * qrow_matmul.h -- C-ABI of libqrow.so, part 3: the product of quantized
 * weight rows with Q8_K activations (128, 64 or 16 values per block), the
 * consumer of both formats.
 *
 * The operation follows this page (cited by title and section):
 *  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …". Section
 *       修复前的数值隐患: the weight codes are multiplied with the 8-bit
 *       activation codes in integer arithmetic and the weight offset is
 *       removed with a per-block sum of the activation codes; stored as
 *       s = d * sum(q) in fp16 (Q8_1), that sum overflows on large
 *       activations. Section 修复方案: Q8_K_128 stores the sum per 32 codes
 *       as an int16 that is not multiplied by d, so the correction is exact
 *       integer arithmetic.
 *
 * Conventions are those of qrow.h (device pointers, 16-byte aligned;
 * asynchronous calls on `stream`; 0 or a negative QR_E* code with nothing
 * launched on failure; nothing allocated).
 */
#ifndef QROW_MATMUL_H
#define QROW_MATMUL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QR_MATMUL_MAX_IN 32768   /* longest row (n_in) */

/*
 * qr_matmul_q8k128 -- y[t][r] = sum_i W[r][i] * A[t][i] [Q8 修复方案].
 *  t      weight type: QR_Q4_0, QR_Q4_1, QR_Q5_0, QR_Q5_1, QR_Q6_0, QR_Q4_K,
 *         QR_Q5_K or QR_Q6_K.
 *  w      packed weight rows [n_out, qr_row_bytes(t, n_in)] (the output of
 *         qr_quantize_rows).
 *  x      packed Q8_K_128 activation rows [n_tok, qr_row_bytes(QR_Q8_K128,
 *         n_in)] (the output of qr_quantize_activations_q8k128).
 *  y      fp32 [n_tok, n_out], written completely.
 * W and A are the values the blocks encode. Per 32 weights the codes are
 * multiplied with the activation codes in int32 (four products per
 * instruction), the weight offset is folded in with the block's int16 code
 * sum (Q4_0, Q5_0, Q6_0: sum(u*q) - 8, 16 or 32 * bsum; Q4_1, Q5_1:
 * m * bsum; Q4_K, Q5_K: dmin*mn_j * bsum_j; Q6_K: the levels are signed,
 * no offset), and the scales are applied in fp32. The fp32 sums are
 * taken in a fixed order (reproducible bit for bit); against the exact
 * product each output is within (n_in/1024 + 9) * 2^-24 of
 * S = sum_i (|scale part_i| + |offset part_i|) * |A[t][i]| ((n_in/512 + 9)
 * for Q6_K, whose 16-weight sub-blocks add two scaled terms per group). From 17 tokens
 * on, the integer products run on the int8 matrix cores (tiles of 64 tokens
 * x 64 rows) and the per-block sums are accumulated in double: each output
 * is then within 2^-24 |y| + 8 * 2^-24 S, inside the same bound.
 * Limits: n_in a positive multiple of 128 (256 for the K types), at most
 * QR_MATMUL_MAX_IN. n_out == 0 or n_tok == 0 is a no-op.
 */
int qr_matmul_q8k128(int t, const void *w, const void *x, int64_t n_out,
                     int64_t n_tok, int64_t n_in, float *y, void *stream);

/*
 * qr_matmul_q8k -- the same product with activations of any Q8_K block size
 * [Q8 技术启示与后续演进: Q8_K64 and Q8_K16 keep Q8_K_128's f32 scale and
 * unscaled int16 code sums]. act is QR_Q8_K128, QR_Q8_K64 or QR_Q8_K16 and x
 * holds [n_tok, qr_row_bytes(act, n_in)] (the output of
 * qr_quantize_activations_q8k). With Q8_K16 each 32-weight group meets two
 * activation blocks: the integer dot product and the offset fold are taken
 * per 16 values and the two scaled terms added in that order, which doubles
 * the fp32 additions per lane: the bound becomes (n_in/512 + 9) * 2^-24 of
 * the same magnitude. From 17 tokens on, Q8_K64 activations take the int8
 * matrix cores like Q8_K_128 (with the same tighter error); Q8_K16 stays
 * on the lane-parallel path. Limits: n_in a positive multiple of the larger
 * of the two block lengths (32 or 256 for the weights), at most
 * QR_MATMUL_MAX_IN; QR_EINVAL_TYPE for an act outside the family.
 */
int qr_matmul_q8k(int t, int act, const void *w, const void *x, int64_t n_out,
                  int64_t n_tok, int64_t n_in, float *y, void *stream);

#ifdef __cplusplus
}
#endif
#endif
