/*
 * matmul_oracle.c -- CPU oracle for the product of quantized weight rows with
 * Q8_K_128 activations (test infrastructure only; see qrow_oracle.c for the
 * rules that apply to the whole oracle).
 *
 * Source, cited by page title and section:
 *  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …". Section
 *       修复前的数值隐患: in the integer dot product of weight codes with 8-bit
 *       activation codes, the offset of the weight codes is removed by
 *       subtracting a per-block sum term; Q8_1 stores that term as s = d *
 *       sum(q) in fp16, which overflows for large activations and makes the
 *       result wrong (NaN). Section 修复方案: Q8_K_128 keeps an fp32 scale per
 *       128 values and an int16 sum per 32 codes that is not multiplied by d,
 *       so the correction cannot overflow.
 *
 * The product is defined plainly: y[t][r] = sum_i w[r][i] * a[t][i], with w
 * and a the exact values the packed blocks encode (Q4_0: d*(u-8); Q5_0:
 * d*(u-16); Q4_1, Q5_1: d*u + m; Q4_K: (d*sc_j)*u - dmin*mn_j; Q6_K:
 * (d*s_j)*(u-32); Q8_K_128 and
 * its 64- and 16-value siblings: d*q), taken in double in ascending i. Each part is exact in double; only
 * the products and the sum round. The oracle also returns
 * S = sum_i (|scale part| + |offset part|) * |a_i|, the magnitude that bounds
 * the rounding error of any float evaluation of the same sum.
 *
 * The Q8_1 comparison (the hazard of [Q8]): activations quantized in
 * 32-value blocks with an fp16 scale d and an fp16 s = d * sum(q), and the
 * asymmetric product evaluated as the pages describe it, the scale part
 * from the integer dot and the offset part from s: per block,
 * d_w * d * sum(u*q) + m * s, in float. When s overflows, so does y.
 */
#include "orc_qrow.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static float rd_f32(const uint8_t *p) { float v; memcpy(&v, p, 4); return v; }
static uint32_t rd_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}
static double rd_f16(const uint8_t *p)
{
    return (double)orc_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
}
/* 6-bit field j of a 6-byte little-endian bit string (field j at bit 6j) */
static int field6(const uint8_t *p, int j)
{
    uint64_t v = 0;
    for (int k = 0; k < 6; ++k)
        v |= (uint64_t)p[k] << (8 * k);
    return (int)((v >> (6 * j)) & 63);
}

/* Level code u of element i (0..31) of a legacy 32-weight block at p. */
static int legacy_code(int type, const uint8_t *p, int i)
{
    if (type == ORC_Q6_0) {
        const uint8_t *qs = p + 12;
        const int lo = i < 16 ? (qs[i] & 15) : (qs[i - 16] >> 4);
        return lo | (((p[4 + i / 4] >> (2 * (i % 4))) & 3) << 4);
    }
    const int sym = type == ORC_Q4_0 || type == ORC_Q5_0;
    const int five = type == ORC_Q5_0 || type == ORC_Q5_1;
    const uint8_t *qh = p + (sym ? 4 : 8);
    const uint8_t *qs = qh + (five ? 4 : 0);
    int u = i < 16 ? (qs[i] & 15) : (qs[i - 16] >> 4);
    if (five)
        u |= (int)((rd_u32(qh) >> i) & 1) << 4;
    return u;
}

/* Exact parts of weight i of a packed row: w_i = a[i] - b[i]. */
static void weight_parts(int type, const uint8_t *row, int64_t n, double *a,
                         double *b)
{
    const int be = orc_block_elems(type);
    const size_t bb = orc_block_bytes(type);
    for (int64_t blk = 0; blk < n / be; ++blk) {
        const uint8_t *p = row + blk * bb;
        for (int i = 0; i < be; ++i) {
            double av = 0.0, bv = 0.0;
            if (type == ORC_Q6_K) {
                const int g = i / 32, k = i % 32;
                const uint8_t *qs = p + 20 + 16 * g;
                int u = k < 16 ? (qs[k] & 15) : (qs[k - 16] >> 4);
                u |= ((p[148 + 8 * g + k / 4] >> (2 * (k % 4))) & 3) << 4;
                const double ds = rd_f16(p) * (double)(int8_t)p[4 + i / 16];
                av = ds * u;
                bv = ds * 32;
            } else if (type == ORC_Q4_K || type == ORC_Q5_K) {
                const int j = i / 32, k = i % 32;
                const uint8_t *qs = p + (type == ORC_Q4_K ? 16 : 48) + 16 * j;
                int u = k < 16 ? (qs[k] & 15) : (qs[k - 16] >> 4);
                if (type == ORC_Q5_K) u |= ((p[16 + 4 * j + k / 8] >> (k % 8)) & 1) << 4;
                av = rd_f16(p) * field6(p + 4, j) * u;
                bv = rd_f16(p + 2) * field6(p + 10, j);
            } else {
                const int sym = type == ORC_Q4_0 || type == ORC_Q5_0 || type == ORC_Q6_0;
                const int five = type == ORC_Q5_0 || type == ORC_Q5_1;
                const double d = rd_f32(p);
                const double m = sym ? 0.0 : rd_f32(p + 4);
                av = d * legacy_code(type, p, i);
                bv = sym ? d * (type == ORC_Q6_0 ? 32 : five ? 16 : 8) : -m;
            }
            a[blk * be + i] = av;
            b[blk * be + i] = bv;
        }
    }
}

/* Exact activation values of a packed row of any Q8_K block size. */
static void act_values(int act_type, const uint8_t *row, int64_t n, double *x)
{
    const int B = orc_block_elems(act_type);
    const size_t ab = orc_block_bytes(act_type);
    for (int64_t blk = 0; blk < n / B; ++blk) {
        const uint8_t *p = row + blk * ab;
        const double d = rd_f32(p);
        for (int i = 0; i < B; ++i)
            x[blk * B + i] = d * (double)(int8_t)p[4 + i];
    }
}

static int is_weight_type(int type)
{
    return type == ORC_Q4_0 || type == ORC_Q4_1 || type == ORC_Q5_0 ||
           type == ORC_Q5_1 || type == ORC_Q4_K || type == ORC_Q6_0 ||
           type == ORC_Q6_K || type == ORC_Q5_K;
}

int orc_matmul_q8k128(int type, const uint8_t *w, const uint8_t *x,
                      int64_t n_out, int64_t n_tok, int64_t n_in, double *y,
                      double *s_abs)
{
    return orc_matmul_q8k(type, ORC_Q8_K128, w, x, n_out, n_tok, n_in, y, s_abs);
}

int orc_matmul_q8k(int type, int act_type, const uint8_t *w, const uint8_t *x,
                   int64_t n_out, int64_t n_tok, int64_t n_in, double *y,
                   double *s_abs)
{
    if (!is_weight_type(type) ||
        (act_type != ORC_Q8_K128 && act_type != ORC_Q8_K64 && act_type != ORC_Q8_K16) ||
        n_out < 0 || n_tok < 0 || n_in <= 0 || n_in % orc_block_elems(act_type) ||
        n_in % orc_block_elems(type))
        return ORC_EINVAL;
    const size_t wrb = orc_row_bytes(type, n_in);
    const size_t xrb = orc_row_bytes(act_type, n_in);
    double *a = malloc(sizeof(double) * n_in);
    double *b = malloc(sizeof(double) * n_in);
    double *xv = malloc(sizeof(double) * n_in * (n_tok > 0 ? n_tok : 1));
    if (!a || !b || !xv) {
        free(a); free(b); free(xv);
        return ORC_EINVAL;
    }
    for (int64_t t = 0; t < n_tok; ++t)
        act_values(act_type, x + t * xrb, n_in, xv + t * n_in);
    for (int64_t r = 0; r < n_out; ++r) {
        weight_parts(type, w + r * wrb, n_in, a, b);
        for (int64_t t = 0; t < n_tok; ++t) {
            const double *xt = xv + t * n_in;
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < n_in; ++i) {
                acc += (a[i] - b[i]) * xt[i];
                mag += (fabs(a[i]) + fabs(b[i])) * fabs(xt[i]);
            }
            y[t * n_out + r] = acc;
            if (s_abs)
                s_abs[t * n_out + r] = mag;
        }
    }
    free(a); free(b); free(xv);
    return ORC_OK;
}

int orc_matmul_q8_1(int type, const uint8_t *w, const float *x, int64_t n_out,
                    int64_t n_tok, int64_t n_in, float *y)
{
    if ((type != ORC_Q4_1 && type != ORC_Q5_1) || n_out < 0 || n_tok < 0 ||
        n_in <= 0 || n_in % 32)
        return ORC_EINVAL;
    const size_t wrb = orc_row_bytes(type, n_in);
    const int64_t ng = n_in / 32;
    float *d16 = malloc(sizeof(float) * ng * (n_tok > 0 ? n_tok : 1));
    float *s16 = malloc(sizeof(float) * ng * (n_tok > 0 ? n_tok : 1));
    int8_t *q = malloc((size_t)n_in * (n_tok > 0 ? n_tok : 1));
    if (!d16 || !s16 || !q) {
        free(d16); free(s16); free(q);
        return ORC_EINVAL;
    }
    /* Q8_1 activations: 32 values, d = amax/127 and s = d*sum(q) in fp16 */
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int64_t g = 0; g < ng; ++g) {
            const float *xg = x + t * n_in + 32 * g;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                amax = fmaxf(amax, fabsf(xg[i]));
            const float d = amax / 127.0f;
            const float id = d > 0.0f ? 1.0f / d : 0.0f;
            int sum = 0;
            for (int i = 0; i < 32; ++i) {
                const int v = (int)rintf(xg[i] * id);
                q[t * n_in + 32 * g + i] = (int8_t)v;
                sum += v;
            }
            d16[t * ng + g] = orc_f16_to_f32(orc_f32_to_f16(d));
            s16[t * ng + g] = orc_f16_to_f32(orc_f32_to_f16(d * (float)sum));
        }
    }
    for (int64_t r = 0; r < n_out; ++r) {
        const uint8_t *row = w + r * wrb;
        for (int64_t t = 0; t < n_tok; ++t) {
            float acc = 0.0f;
            for (int64_t g = 0; g < ng; ++g) {
                const uint8_t *p = row + g * orc_block_bytes(type);
                const float dw = rd_f32(p), m = rd_f32(p + 4);
                int iu = 0;                 /* integer dot of codes */
                for (int i = 0; i < 32; ++i)
                    iu += legacy_code(type, p, i) * q[t * n_in + 32 * g + i];
                acc += dw * d16[t * ng + g] * (float)iu + m * s16[t * ng + g];
            }
            y[t * n_out + r] = acc;
        }
    }
    free(d16); free(s16); free(q);
    return ORC_OK;
}
