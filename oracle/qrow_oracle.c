/*
 * qrow_oracle.c -- CPU oracle for importance-matrix-weighted row quantization.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, single-threaded reference
 * that the GPU library is checked against. Only the test-suite, the package
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * code, header, table or constant generator with the GPU library.
 *
 * Sources, cited by page title and section:
 *  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
 *       的由来与原理". Section 一 gives the row statistic sigma2 (mean of x^2
 *       over the whole row), the element weight qw*sqrt(sigma2 + x^2), and the
 *       block routine: weighted least-squares scale sumlx/suml2 followed by
 *       greedy level flips along g = scale*w*(x - scale*l). Section 三 gives
 *       the asymptotics of the sqrt term.
 *  [KQ] "3.2 K-quants 与重要性矩阵：量化兵器谱", section 一: the Q4_K super-block
 *       (256 weights = 8 sub-blocks, 6-bit sub-scales, fp16 super-scale,
 *       about 4.5 bits per weight).
 *  [LQ] "从零理解 LLM 量化 PTQ、QAT 与 ik_llama.cpp 量化体系的源码级导学",
 *       section 2.1: the legacy 32-weight blocks Q4_0, Q4_1, Q5_0, Q5_1.
 *  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …", section
 *       修复方案: the Q8_K_128 block (128 values, fp32 scale, int8 codes, an
 *       int16 sum per 32 codes that is not multiplied by the scale).
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * The pages' block routine works in single precision (its snippet declares
 * the row sum, sigma2 and the returned scale as float); every per-element and
 * per-block sum here is therefore a float sum taken in ascending element
 * order. Two readings depart from plain float: the row sum of x^2 is taken in
 * double (so that its value does not depend on the order of summation) and
 * the comparisons of trial-scale scores and the asymmetric two-parameter
 * solve are done in double.
 */
#include "orc_qrow.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define MAXN 256

/* Trial-scale offsets, in units of ORC_CAND_STEP levels, in trial order. */
static const int cand_offset[5] = {0, -1, 1, -2, 2};

void orc_solver_constants(int32_t *c)
{
    c[0] = (int32_t)(ORC_CAND_STEP * 4.0f);
    c[1] = ORC_SYM_CAND;
    c[2] = ORC_SYM_FLIP_PASSES;
    c[3] = ORC_ASYM_CAND;
    c[4] = ORC_ASYM_FLIP_PASSES;
    c[5] = MAXN;
}

/* ------------------------------------------------------------------------ */
/* formats                                                                   */

int orc_block_elems(int type)
{
    switch (type) {
    case ORC_Q4_0: case ORC_Q4_1: case ORC_Q5_0: case ORC_Q5_1: case ORC_Q6_0: return 32;
    case ORC_Q4_K: case ORC_Q5_K: case ORC_Q6_K: return 256;
    case ORC_Q8_K128: return 128;
    case ORC_Q8_K64: return 64;
    case ORC_Q8_K16: return 16;
    default: return 0;
    }
}

size_t orc_block_bytes(int type)
{
    switch (type) {
    case ORC_Q4_0: return 4 + 16;            /* d, 32 nibbles            */
    case ORC_Q4_1: return 4 + 4 + 16;        /* d, m, 32 nibbles         */
    case ORC_Q5_0: return 4 + 4 + 16;        /* d, 5th-bit plane, nibbles */
    case ORC_Q5_1: return 4 + 4 + 4 + 16;    /* d, m, 5th bits, nibbles  */
    case ORC_Q4_K: return 2 + 2 + 6 + 6 + 128; /* d16, dmin16, sc6, mn6, qs */
    case ORC_Q8_K128: return 4 + 128 + 8;    /* d, int8 x128, int16 x4   */
    case ORC_Q6_0: return 4 + 8 + 16;        /* d, 2-bit plane, nibbles  */
    case ORC_Q8_K64: return 4 + 64 + 4;      /* d, int8 x64, int16 x2    */
    case ORC_Q8_K16: return 4 + 16 + 2 + 2;  /* d, int8 x16, int16, pad  */
    case ORC_Q6_K: return 2 + 2 + 16 + 128 + 64; /* d16, pad, sc, nibbles, planes */
    case ORC_Q5_K: return 2 + 2 + 6 + 6 + 32 + 128; /* d16, dmin16, sc6, mn6, 5th bits, qs */
    default: return 0;
    }
}

size_t orc_row_bytes(int type, int64_t n_per_row)
{
    int be = orc_block_elems(type);
    if (be == 0 || n_per_row < 0 || n_per_row % be != 0) return 0;
    return (size_t)(n_per_row / be) * orc_block_bytes(type);
}

static void put_f32(uint8_t *p, float v) { memcpy(p, &v, 4); }
static float get_f32(const uint8_t *p) { float v; memcpy(&v, p, 4); return v; }
static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}
static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
           ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 (written from the format's definition)                  */

uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return 0x7e00;
    if (isinf(f)) return (uint16_t)(sign | 0x7c00);
    if (a == 0.0) return sign;
    /* Spacing of binary16 values near a: 2^-24 below 2^-14 (subnormals),
     * otherwise 2^(e-10) where 2^e <= a < 2^(e+1). */
    int e;
    frexp(a, &e);                 /* a = m * 2^e, 0.5 <= m < 1 */
    e -= 1;                       /* now 2^e <= a < 2^(e+1)     */
    if (e < -14) e = -14;
    double spacing = ldexp(1.0, e - 10);
    double k = rint(a / spacing);   /* exact division by a power of two */
    double v = k * spacing;         /* the nearest binary16 value (ties even) */
    if (v >= 65520.0 || v > 65504.0) return (uint16_t)(sign | 0x7c00);
    if (v < ldexp(1.0, -14))        /* subnormal: mantissa counts 2^-24 */
        return (uint16_t)(sign | (uint16_t)rint(v / ldexp(1.0, -24)));
    int ev;
    frexp(v, &ev);
    ev -= 1;                        /* 2^ev <= v < 2^(ev+1) */
    uint16_t mant = (uint16_t)rint(v / ldexp(1.0, ev - 10)) - 1024;
    return (uint16_t)(sign | (uint16_t)((ev + 15) << 10) | mant);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
    double v;
    if (ex == 31) v = man ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)man, -24);
    else v = ldexp((double)(man + 1024), ex - 25);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* row statistic and element importances [WT §一]                            */

double orc_row_sigma2_f64(const float *x, int64_t n)
{
    /* Reading: the sum of squares is accumulated in double. Each x*x of a
     * float is exact in double, so only the additions round, and the final
     * float value does not depend on the order of summation except when the
     * double sum lies within a few units of its last place of a float
     * rounding boundary. */
    double acc = 0.0;
    for (int64_t j = 0; j < n; ++j) acc += (double)x[j] * (double)x[j];
    return acc / (double)n;
}

float orc_row_sigma2(const float *x, int64_t n)
{
    return (float)orc_row_sigma2_f64(x, n);
}

/* The magnitude factor of element importance under each weighting
 * [WT 一, 二]: the pages' sqrt(sigma2 + x^2), and the forms that section
 * lists as tried before it (x^2, |x|, sigma2 + x^2, sigma + |x|) and the
 * imatrix alone (factor 1). Reading: sigma2 + x^2 is one fused operation in
 * both forms that use it, sigma = sqrtf(sigma2) correctly rounded. */
static float magnitude(float x, float sigma2, float sigma, int mode)
{
    switch (mode) {
    case ORC_W_X2:              return x * x;
    case ORC_W_ABS_X:           return fabsf(x);
    case ORC_W_SIGMA2_PLUS_X2:  return fmaf(x, x, sigma2);
    case ORC_W_SIGMA_PLUS_ABS_X: return sigma + fabsf(x);
    case ORC_W_IMATRIX_ONLY:    return 1.0f;
    default:                    return sqrtf(fmaf(x, x, sigma2));
    }
}

void orc_row_weights_mode(const float *x, const float *q, int64_t n,
                          float sigma2, int mode, float *w)
{
    if (mode == ORC_W_SQRT_SIGMA2_X2) {
        orc_row_weights(x, q, n, sigma2, w);
        return;
    }
    const float sigma = sqrtf(sigma2);
    for (int64_t j = 0; j < n; ++j) {
        const float m = magnitude(x[j], sigma2, sigma, mode);
        w[j] = q ? q[j] * m : m;
    }
}

void orc_row_weights(const float *x, const float *q, int64_t n, float sigma2,
                     float *w)
{
    /* w_j = qw_j * sqrt(sigma2 + x_j^2) [WT §一]. qw_j is the importance of
     * element j's own column: the pages' snippet elides the block offset of
     * qw, and the text says the importance corresponds one-to-one to the
     * element. Reading: sigma2 + x^2 is one fused operation (one rounding)
     * and the square root is correctly rounded. q == NULL means qw = 1. */
    for (int64_t j = 0; j < n; ++j) {
        float s = sqrtf(fmaf(x[j], x[j], sigma2));
        w[j] = q ? q[j] * s : s;
    }
}

/* ------------------------------------------------------------------------ */
/* helpers                                                                   */

static float clampf(float v, float lo, float hi)
{
    return fminf(fmaxf(v, lo), hi);
}

/* Greedy level flips on one block [WT §一].
 *
 * The block is fitted as y_j ~ d * l_j with d = A / B, where
 * A = sum w_j y_j l_j and B = sum w_j l_j^2 (the pages' sumlx and suml2).
 * Each pass visits j = 0 .. n-1 in order. The pages' gradient is
 * g_j = d * w_j * (y_j - d * l_j); a flip moves l_j one level along
 * s = sign(g_j). With d = A / B and B > 0 that sign is sign(A) * sign(e_j),
 * e_j = y_j * B - l_j * A, so no division is needed. After the move the sums
 * are A' = A + s*w_j*y_j and B' = B + w_j*(2*s*l_j + 1). The flip is kept
 * only if the least-squares error with d refitted strictly drops, i.e. the
 * score A^2/B strictly rises: A'^2 * B > A^2 * B' with B' > 0, compared by
 * cross multiplication in the operation order below. Reading: the pages give
 * no pass count; ORC_*_FLIP_PASSES passes are run, stopping after a pass that
 * accepts nothing (a pass with no change would repeat exactly). */
static void flip_passes(int n, const float *y, const float *w, const float *wy,
                        float lo_level, float hi_level, int F, float *L,
                        float *A_io, float *B_io, int32_t *info)
{
    float A = *A_io, B = *B_io;
    int accepted = 0, passes = 0, converged = 0;
    for (int p = 0; p < F; ++p) {
        int changed = 0;
        ++passes;
        for (int j = 0; j < n; ++j) {
            float t = L[j] * A;
            float e = fmaf(y[j], B, -t);
            float s = ((signbit(A) != 0) != (signbit(e) != 0)) ? -1.0f : 1.0f;
            float lp = L[j] + s;
            float A1 = fmaf(s, wy[j], A);
            float B1 = fmaf(w[j], fmaf(2.0f * s, L[j], 1.0f), B);
            int better = (A1 * A1) * B > (A * A) * B1;
            if (better && B1 > 0.0f && lp >= lo_level && lp <= hi_level) {
                A = A1;
                B = B1;
                L[j] = lp;
                changed = 1;
                ++accepted;
            }
        }
        if (!changed) { converged = 1; break; }
    }
    *A_io = A;
    *B_io = B;
    if (info) { info[1] = accepted; info[2] = passes; info[3] = converged; }
}

/* ------------------------------------------------------------------------ */
/* symmetric block: levels -nmax .. nmax-1, one scale [WT §一]                */

int orc_solve_sym(int n, const float *x, const float *w, int nmax, int K, int F,
                  int8_t *l_out, float *d_out, int32_t *info)
{
    if (n < 1 || n > MAXN || nmax < 1 || K < 1 || K > 5 || F < 0) return ORC_EINVAL;
    float L[MAXN], wx[MAXN];
    const float lo_level = (float)-nmax, hi_level = (float)(nmax - 1);
    int32_t inf_local[4] = {-1, 0, 0, 1};

    /* The element of largest magnitude; the first one on ties (reading). */
    int imax = 0;
    float amax = fabsf(x[0]);
    for (int i = 1; i < n; ++i)
        if (fabsf(x[i]) > amax) { amax = fabsf(x[i]); imax = i; }
    const float xm = x[imax];

    for (int i = 0; i < n; ++i) wx[i] = w[i] * x[i];

    /* Trial scales (reading; the pages name the least-squares scale and the
     * flips but not the start): the largest-magnitude element is mapped to
     * the long end -c of the level range, c = nmax + 0.25*k, k taken in the
     * order 0, -1, +1, -2, +2. Each trial rounds every element to the
     * nearest level, clamps, and scores its least-squares fit by
     * sumlx^2 / suml2 (the error is sum w x^2 minus that score). The best
     * score wins; an earlier trial wins ties. Scores are compared by cross
     * multiplication in double. */
    int best = -1;
    float bS1 = 0.0f, bS2 = 0.0f, bis = 0.0f;
    if (amax > 0.0f) {
        for (int k = 0; k < K; ++k) {
            float c = (float)nmax + ORC_CAND_STEP * (float)cand_offset[k];
            float is = -c / xm;
            if (!isfinite(is)) continue;
            float S1 = 0.0f, S2 = 0.0f;
            for (int i = 0; i < n; ++i) {
                float l = clampf(rintf(x[i] * is), lo_level, hi_level);
                S1 = fmaf(wx[i], l, S1);
                S2 = fmaf(w[i] * l, l, S2);
            }
            if (!(S2 > 0.0f)) continue;
            int better = 0;
            if (best < 0) {
                better = 1;
            } else {
                double lhs = ((double)S1 * (double)S1) * (double)bS2;
                double rhs = ((double)bS1 * (double)bS1) * (double)S2;
                better = lhs > rhs;
            }
            if (better) { best = k; bS1 = S1; bS2 = S2; bis = is; }
        }
    }

    if (best < 0) {
        /* Zero block: all-zero input, a scale that is not finite, or no
         * weight on the block. */
        for (int i = 0; i < n; ++i) l_out[i] = 0;
        *d_out = 0.0f;
        if (info) { info[0] = -1; info[1] = 0; info[2] = 0; info[3] = 1; }
        return ORC_OK;
    }

    for (int i = 0; i < n; ++i) L[i] = clampf(rintf(x[i] * bis), lo_level, hi_level);
    float A = bS1, B = bS2;
    inf_local[0] = best;
    flip_passes(n, x, w, wx, lo_level, hi_level, F, L, &A, &B, inf_local);

    *d_out = A / B;
    for (int i = 0; i < n; ++i) l_out[i] = (int8_t)L[i];
    if (info) memcpy(info, inf_local, sizeof inf_local);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* non-negative values, levels 0 .. nmax, one scale: the Q4_K sub-scales      */

/* Weighted fit of n values v_j >= 0 as v_j ~ d * l_j, l_j in 0..nmax, with
 * weights W_j: the least-squares scale and greedy flips of [WT 一] applied
 * to the eight sub-scales (or sub-offsets) of a Q4_K super-block.
 * Readings (the pages fix the sub-scales' width, not how they are chosen):
 * the trial scales map the largest value to the top of the level range,
 * is = c / max v with c = nmax + 0.25*k, k in the order 0, -1, +1, -2, +2
 * (the symmetric blocks' schedule, mirrored to the positive end); each
 * trial rounds v_j * is to the nearest level in float and clamps. Because
 * one sub-block can carry most of the weight, the fit's error is a small
 * difference of large scores, so the sums sumlx = sum W v l and
 * suml2 = sum W l^2, the score comparisons (by cross multiplication, an
 * earlier trial winning ties) and the flips (the rule of flip_passes(),
 * element by element in order) are evaluated in double; d = sumlx/suml2
 * rounded once to float. All-zero values, a scale that is not finite or no
 * weight give levels 0 and d = 0. */
int orc_fit_levels_pos(int n, const float *v, const float *W, int nmax, int K,
                       int F, uint8_t *l_out, float *d_out, int32_t *info)
{
    if (n < 1 || n > MAXN || nmax < 1 || K < 1 || K > 5 || F < 0) return ORC_EINVAL;
    float L[MAXN];
    double Wv[MAXN];
    const float hi_level = (float)nmax;
    int32_t inf_local[4] = {-1, 0, 0, 1};
    float vmax = v[0];
    for (int i = 1; i < n; ++i) vmax = fmaxf(vmax, v[i]);
    for (int i = 0; i < n; ++i) Wv[i] = (double)W[i] * (double)v[i];   /* exact */

    int best = -1;
    double bS1 = 0.0, bS2 = 0.0;
    float bis = 0.0f;
    if (vmax > 0.0f) {
        for (int k = 0; k < K; ++k) {
            float c = (float)nmax + ORC_CAND_STEP * (float)cand_offset[k];
            float is = c / vmax;
            if (!isfinite(is)) continue;
            double S1 = 0.0, S2 = 0.0;
            for (int i = 0; i < n; ++i) {
                double l = (double)clampf(rintf(v[i] * is), 0.0f, hi_level);
                S1 = fma(Wv[i], l, S1);
                S2 = fma((double)W[i] * l, l, S2);
            }
            if (!(S2 > 0.0)) continue;
            if (best < 0 || (S1 * S1) * bS2 > (bS1 * bS1) * S2) {
                best = k; bS1 = S1; bS2 = S2; bis = is;
            }
        }
    }
    if (best < 0) {
        for (int i = 0; i < n; ++i) l_out[i] = 0;
        *d_out = 0.0f;
        if (info) { info[0] = -1; info[1] = 0; info[2] = 0; info[3] = 1; }
        return ORC_OK;
    }
    for (int i = 0; i < n; ++i) L[i] = clampf(rintf(v[i] * bis), 0.0f, hi_level);
    double A = bS1, B = bS2;
    int accepted = 0, passes = 0, converged = 0;
    for (int p = 0; p < F; ++p) {
        int changed = 0;
        ++passes;
        for (int j = 0; j < n; ++j) {
            double e = fma((double)v[j], B, -((double)L[j] * A));
            double s = ((signbit(A) != 0) != (signbit(e) != 0)) ? -1.0 : 1.0;
            double lp = (double)L[j] + s;
            double A1 = fma(s, Wv[j], A);
            double B1 = fma((double)W[j], fma(2.0 * s, (double)L[j], 1.0), B);
            if ((A1 * A1) * B > (A * A) * B1 && B1 > 0.0 && lp >= 0.0 && lp <= (double)nmax) {
                A = A1;
                B = B1;
                L[j] = (float)lp;
                changed = 1;
                ++accepted;
            }
        }
        if (!changed) { converged = 1; break; }
    }
    inf_local[0] = best;
    inf_local[1] = accepted;
    inf_local[2] = passes;
    inf_local[3] = converged;
    *d_out = (float)(A / B);
    for (int i = 0; i < n; ++i) l_out[i] = (uint8_t)L[i];
    if (info) memcpy(info, inf_local, sizeof inf_local);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* asymmetric block: levels 0 .. nmax, scale and offset, x ~ d*l + m          */

/* Weighted least squares for (d, m) from the five block sums, in double.
 * The reconstruction error is sum w x^2 minus the returned score.
 * Reading: codes whose weighted spread is below 2^-16 of sum w l^2 are
 * treated as constant (d = 0, m = weighted mean). The sums arrive as floats,
 * so D = Sw*Sll - Sl^2 carries an error of a few 2^-24 of Sw*Sll; below
 * 2^-16 of it the solved (d, m) would rest on fewer than six good bits.
 * With k4, a positive offset is replaced by the best fit with m = 0. */
static void fit_dm(float Sw_, float Sx_, float Sl_, float Sll_, float Slx_,
                   int k4, double *d, double *m, double *score)
{
    double Sw = Sw_, Sx = Sx_, Sl = Sl_, Sll = Sll_, Slx = Slx_;
    double D = Sw * Sll - Sl * Sl;
    double dd, mm;
    if (D > Sw * Sll * 0x1p-16) {
        double r = 1.0 / D;
        dd = (Sw * Slx - Sl * Sx) * r;
        mm = (Sll * Sx - Sl * Slx) * r;
    } else {
        dd = 0.0;
        mm = Sx / Sw;
    }
    if (k4 && mm > 0.0) {
        mm = 0.0;
        dd = Sll > 0.0 ? Slx / Sll : 0.0;
    }
    *d = dd;
    *m = mm;
    *score = dd * Slx + mm * Sx;
}

static void asym_sums(int n, const float *w, const float *wx, const float *L,
                      float *Sl, float *Sll, float *Slx)
{
    float a = 0.0f, b = 0.0f, c = 0.0f;
    for (int i = 0; i < n; ++i) {
        float wl = w[i] * L[i];
        a = a + wl;
        b = fmaf(wl, L[i], b);
        c = fmaf(wx[i], L[i], c);
    }
    *Sl = a; *Sll = b; *Slx = c;
}

int orc_solve_asym(int n, const float *x, const float *w, int nmax, int K,
                   int F, int k4, uint8_t *l_out, float *d_out, float *m_out,
                   int32_t *info)
{
    if (n < 1 || n > MAXN || nmax < 1 || K < 1 || K > 5 || F < 0) return ORC_EINVAL;
    float L[MAXN], wx[MAXN], xs[MAXN], y[MAXN], wy[MAXN];
    const float lo_level = 0.0f, hi_level = (float)nmax;
    int32_t inf_local[4] = {-1, 0, 0, 1};

    /* Range of the block. Adding +0 turns a -0 bound into +0, so the result
     * does not depend on which of two equal zeros fminf/fmaxf return. */
    float lo = x[0], hi = x[0];
    for (int i = 1; i < n; ++i) { lo = fminf(lo, x[i]); hi = fmaxf(hi, x[i]); }
    lo = lo + 0.0f;
    hi = hi + 0.0f;
    if (k4) lo = fminf(lo, 0.0f);  /* Q4_K stores the offset as -dmin*mn, mn >= 0 */

    float Sw = 0.0f, Sx = 0.0f;
    for (int i = 0; i < n; ++i) {
        wx[i] = w[i] * x[i];
        xs[i] = x[i] - lo;
        Sw = Sw + w[i];
        Sx = Sx + wx[i];
    }

    if (hi == lo || !(Sw > 0.0f)) {
        /* Constant block, or no weight: offset only. */
        for (int i = 0; i < n; ++i) l_out[i] = 0;
        *d_out = 0.0f;
        *m_out = lo;
        if (info) { info[0] = -1; info[1] = 0; info[2] = 0; info[3] = 1; }
        return ORC_OK;
    }

    /* Trial scales (reading): is = (nmax + 0.25*k) / (hi - lo), k taken in
     * the order 0, -1, +1; l = clamp(rint((x - lo) * is), 0, nmax); each
     * trial is scored by its two-parameter least-squares fit. */
    const float range = hi - lo;
    int best = -1;
    float bis = 0.0f, bSl = 0.0f, bSll = 0.0f, bSlx = 0.0f;
    double bm = 0.0, bscore = 0.0;
    for (int k = 0; k < K; ++k) {
        float is = ((float)nmax + ORC_CAND_STEP * (float)cand_offset[k]) / range;
        if (!isfinite(is)) continue;
        for (int i = 0; i < n; ++i) L[i] = clampf(rintf(xs[i] * is), lo_level, hi_level);
        float Sl, Sll, Slx;
        asym_sums(n, w, wx, L, &Sl, &Sll, &Slx);
        double d, m, score;
        fit_dm(Sw, Sx, Sl, Sll, Slx, k4, &d, &m, &score);
        if (best < 0 || score > bscore) {
            best = k; bis = is; bm = m; bscore = score;
            bSl = Sl; bSll = Sll; bSlx = Slx;
        }
    }
    if (best < 0) {
        for (int i = 0; i < n; ++i) l_out[i] = 0;
        *d_out = 0.0f;
        *m_out = lo;
        if (info) { info[0] = -1; info[1] = 0; info[2] = 0; info[3] = 1; }
        return ORC_OK;
    }

    for (int i = 0; i < n; ++i) L[i] = clampf(rintf(xs[i] * bis), lo_level, hi_level);

    /* Flips (reading): the offset m of the winning trial is held fixed and
     * the scale-only rule of flip_passes() is applied to y = x - m, starting
     * from A = sum w y l = Slx - m*Sl and B = sum w l^2 = Sll of that trial;
     * the pass keeps A and B as running sums, move by move. Then (d, m) are
     * refitted jointly on the final levels from the sums the pass kept:
     * Sll = B and Slx = A + m*Sl (equal, in exact arithmetic, to the sums
     * recomputed from the final codes), with Sl summed again. */
    const float mf = (float)bm;
    for (int i = 0; i < n; ++i) {
        y[i] = x[i] - mf;
        wy[i] = w[i] * y[i];
    }
    float A = fmaf(-mf, bSl, bSlx), B = bSll;
    inf_local[0] = best;
    flip_passes(n, y, w, wy, lo_level, hi_level, F, L, &A, &B, inf_local);

    float Sl = 0.0f;
    for (int i = 0; i < n; ++i) Sl = Sl + w[i] * L[i];
    const float Sll = B, Slx = fmaf(mf, Sl, A);
    double d, m, score;
    fit_dm(Sw, Sx, Sl, Sll, Slx, k4, &d, &m, &score);

    *d_out = (float)d;
    *m_out = (float)m;
    for (int i = 0; i < n; ++i) l_out[i] = (uint8_t)L[i];
    if (info) memcpy(info, inf_local, sizeof inf_local);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* block packers                                                              */

/* 32 codes u_i in [0, 15]: byte i holds u_i (low nibble) and u_{i+16}
 * (high nibble). */
static void pack_nibbles32(const uint8_t *u, uint8_t *qs)
{
    for (int i = 0; i < 16; ++i)
        qs[i] = (uint8_t)((u[i] & 15) | ((u[i + 16] & 15) << 4));
}

static uint32_t pack_high_bits32(const uint8_t *u)
{
    uint32_t qh = 0;
    for (int i = 0; i < 32; ++i) qh |= (uint32_t)((u[i] >> 4) & 1) << i;
    return qh;
}

/* The two high bits of the 6-bit codes: bits 2i, 2i+1 of a 64-bit
 * little-endian plane hold bits 4 and 5 of u_i. */
static void pack_plane2(const uint8_t *u, uint8_t *qh)
{
    uint64_t v = 0;
    for (int i = 0; i < 32; ++i) v |= (uint64_t)((u[i] >> 4) & 3) << (2 * i);
    for (int k = 0; k < 8; ++k) qh[k] = (uint8_t)(v >> (8 * k));
}

static void quantize_block32(int type, const float *x, const float *w, uint8_t *out)
{
    uint8_t u[32];
    if (type == ORC_Q6_0) {
        /* [WT 一]: the same symmetric routine on 6-bit levels -32..31 */
        int8_t l[32];
        float d;
        orc_solve_sym(32, x, w, 32, ORC_SYM_CAND, ORC_SYM_FLIP_PASSES, l, &d, NULL);
        for (int i = 0; i < 32; ++i) u[i] = (uint8_t)(l[i] + 32);
        put_f32(out, d);
        pack_plane2(u, out + 4);
        pack_nibbles32(u, out + 12);
    } else if (type == ORC_Q4_0 || type == ORC_Q5_0) {
        int nmax = type == ORC_Q4_0 ? 8 : 16;
        int8_t l[32];
        float d;
        orc_solve_sym(32, x, w, nmax, ORC_SYM_CAND, ORC_SYM_FLIP_PASSES, l, &d, NULL);
        for (int i = 0; i < 32; ++i) u[i] = (uint8_t)(l[i] + nmax);
        put_f32(out, d);
        if (type == ORC_Q4_0) {
            pack_nibbles32(u, out + 4);
        } else {
            put_u32(out + 4, pack_high_bits32(u));
            pack_nibbles32(u, out + 8);
        }
    } else {
        int nmax = type == ORC_Q4_1 ? 15 : 31;
        float d, m;
        orc_solve_asym(32, x, w, nmax, ORC_ASYM_CAND, ORC_ASYM_FLIP_PASSES, 0, u, &d, &m, NULL);
        put_f32(out, d);
        put_f32(out + 4, m);
        if (type == ORC_Q4_1) {
            pack_nibbles32(u, out + 8);
        } else {
            put_u32(out + 8, pack_high_bits32(u));
            pack_nibbles32(u, out + 12);
        }
    }
}

/* 8 six-bit values into 6 bytes, value j at bit 6j, little-endian. */
static void pack6x8(const uint8_t *v, uint8_t *p)
{
    uint64_t bits = 0;
    for (int j = 0; j < 8; ++j) bits |= (uint64_t)(v[j] & 63) << (6 * j);
    for (int b = 0; b < 6; ++b) p[b] = (uint8_t)(bits >> (8 * b));
}

static void unpack6x8(const uint8_t *p, uint8_t *v)
{
    uint64_t bits = 0;
    for (int b = 0; b < 6; ++b) bits |= (uint64_t)p[b] << (8 * b);
    for (int j = 0; j < 8; ++j) v[j] = (uint8_t)((bits >> (6 * j)) & 63);
}

/* Q4_K super-block [KQ §一]: 8 sub-blocks of 32, each fitted as
 * x ~ a_j * l - b_j with levels 0..nmax (15). Q5_K is the same
 * super-block with levels 0..31 (nmax = 31; [LQ] 2.2 lists Q5_K among the
 * K-quants and [KQ] names Q5_K_M among the 4-bit-and-above K choices, with
 * no layout; the layout is this library's): the fifth bit
 * of the levels of sub-block j is a 32-bit word at byte 16 + 4 j (bit i for
 * element i) and the low nibbles follow at byte 48 + 16 j.
 * Readings, fit == ORC_FIT_MAX (the
 * default): the super-scales are d = fp16(max a_j / 63) and
 * dmin = fp16(max b_j / 63) (round to nearest even, subnormals kept);
 * sub-scales are sc_j = rint(a_j / d) and mn_j = rint(b_j / dmin) clamped to
 * 0..63. fit == ORC_FIT_WEIGHTED: the 6-bit sub-scales and sub-offsets are
 * each fitted by orc_fit_levels_pos() with weight W_j = the sum of the
 * sub-block's 32 importances (ascending order), d and dmin = fp16 of the
 * fitted scales, sc_j and mn_j = the fitted levels (0 where the fp16 scale
 * is 0). Either way the levels are then re-rounded against the stored
 * scales so that the decoder reproduces the fit. */
static void quantize_kquant(const float *x, const float *w, int fit, int nmax, uint8_t *out)
{
    float a[8], b[8], W[8];
    for (int j = 0; j < 8; ++j) {
        uint8_t l[32];
        float d, m;
        orc_solve_asym(32, x + 32 * j, w + 32 * j, nmax, ORC_ASYM_CAND,
                       ORC_ASYM_FLIP_PASSES, 1, l, &d, &m, NULL);
        a[j] = d > 0.0f ? d : 0.0f;
        b[j] = -m > 0.0f ? -m : 0.0f;
        float sw = 0.0f;
        for (int i = 0; i < 32; ++i) sw = sw + w[32 * j + i];
        W[j] = sw;
    }
    uint16_t d16, m16;
    uint8_t sc[8], mn[8];
    if (fit == ORC_FIT_WEIGHTED) {
        float da, db;
        orc_fit_levels_pos(8, a, W, 63, ORC_SYM_CAND, ORC_SYM_FLIP_PASSES, sc, &da, NULL);
        orc_fit_levels_pos(8, b, W, 63, ORC_SYM_CAND, ORC_SYM_FLIP_PASSES, mn, &db, NULL);
        d16 = orc_f32_to_f16(da);
        m16 = orc_f32_to_f16(db);
        for (int j = 0; j < 8; ++j) {
            if (orc_f16_to_f32(d16) == 0.0f) sc[j] = 0;
            if (orc_f16_to_f32(m16) == 0.0f) mn[j] = 0;
        }
    } else {
        float amx = a[0], bmx = b[0];
        for (int j = 1; j < 8; ++j) { amx = fmaxf(amx, a[j]); bmx = fmaxf(bmx, b[j]); }
        d16 = orc_f32_to_f16(amx / 63.0f);
        m16 = orc_f32_to_f16(bmx / 63.0f);
        float dA0 = orc_f16_to_f32(d16), dB0 = orc_f16_to_f32(m16);
        for (int j = 0; j < 8; ++j) {
            sc[j] = dA0 > 0.0f ? (uint8_t)clampf(rintf(a[j] / dA0), 0.0f, 63.0f) : 0;
            mn[j] = dB0 > 0.0f ? (uint8_t)clampf(rintf(b[j] / dB0), 0.0f, 63.0f) : 0;
        }
    }
    float dA = orc_f16_to_f32(d16), dB = orc_f16_to_f32(m16);
    out[0] = (uint8_t)d16; out[1] = (uint8_t)(d16 >> 8);
    out[2] = (uint8_t)m16; out[3] = (uint8_t)(m16 >> 8);
    pack6x8(sc, out + 4);
    pack6x8(mn, out + 10);
    for (int j = 0; j < 8; ++j) {
        float ds = dA * (float)sc[j];   /* exact: 11-bit times 6-bit */
        float dm = dB * (float)mn[j];
        uint8_t u[32];
        if (ds == 0.0f) {
            memset(u, 0, sizeof u);
        } else {
            float id = 1.0f / ds;
            for (int i = 0; i < 32; ++i)
                u[i] = (uint8_t)clampf(rintf((x[32 * j + i] + dm) * id), 0.0f, (float)nmax);
        }
        if (nmax == 15) {
            pack_nibbles32(u, out + 16 + 16 * j);
        } else {
            uint32_t qh = 0;
            for (int i = 0; i < 32; ++i) qh |= (uint32_t)((u[i] >> 4) & 1) << i;
            for (int k = 0; k < 4; ++k) out[16 + 4 * j + k] = (uint8_t)(qh >> (8 * k));
            uint8_t lo[32];
            for (int i = 0; i < 32; ++i) lo[i] = u[i] & 15;
            pack_nibbles32(lo, out + 48 + 16 * j);
        }
    }
}

/* Q6_K super-block: the two-level scaling of [KQ 一] for 6-bit levels.
 * Readings (the pages describe the K-quant structure through Q4_K and name
 * the 6-bit tier without its layout): 256 weights in 16 sub-blocks of 16;
 * each sub-block fitted by the symmetric routine [WT 一] on levels
 * -32..31, giving a signed scale d_j; the super-scale d = fp16(max |d_j| /
 * 127) (round to nearest even, subnormals kept); signed 8-bit sub-scales
 * s_j = rint(d_j / d) clamped to -127..127 (0 when d is 0); the levels are
 * then re-rounded against the stored scale d*s_j (exact in float) and
 * stored as u = l + 32. Layout: f16 d | 2 zero bytes | i8 s[16] | nibbles
 * of the eight 32-weight groups (16 B each, u_i low, u_{i+16} high) | the
 * 2-bit planes of the eight groups (8 B each, bits 2i, 2i+1 = bits 4, 5 of
 * u_i). */
static void quantize_q6k(const float *x, const float *w, uint8_t *out)
{
    float dj[16];
    for (int j = 0; j < 16; ++j) {
        int8_t l[16];
        orc_solve_sym(16, x + 16 * j, w + 16 * j, 32, ORC_SYM_CAND,
                      ORC_SYM_FLIP_PASSES, l, &dj[j], NULL);
    }
    float amx = 0.0f;
    for (int j = 0; j < 16; ++j) amx = fmaxf(amx, fabsf(dj[j]));
    uint16_t d16 = orc_f32_to_f16(amx / 127.0f);
    float dA = orc_f16_to_f32(d16);
    int8_t sc[16];
    for (int j = 0; j < 16; ++j)
        sc[j] = dA > 0.0f ? (int8_t)clampf(rintf(dj[j] / dA), -127.0f, 127.0f) : 0;
    uint8_t u[256];
    for (int j = 0; j < 16; ++j) {
        float ds = dA * (float)sc[j];   /* exact: 11-bit times 8-bit */
        if (ds == 0.0f) {
            memset(u + 16 * j, 32, 16);
        } else {
            float id = 1.0f / ds;
            for (int i = 0; i < 16; ++i)
                u[16 * j + i] = (uint8_t)(clampf(rintf(x[16 * j + i] * id), -32.0f, 31.0f) + 32.0f);
        }
    }
    out[0] = (uint8_t)d16; out[1] = (uint8_t)(d16 >> 8);
    out[2] = 0; out[3] = 0;
    memcpy(out + 4, sc, 16);
    for (int g = 0; g < 8; ++g) {
        pack_nibbles32(u + 32 * g, out + 20 + 16 * g);
        pack_plane2(u + 32 * g, out + 148 + 8 * g);
    }
}

/* ------------------------------------------------------------------------ */
/* row drivers                                                                */

static int quantize_row_impl(int type, const float *x, const float *q,
                             int64_t n, float sigma2, int mode, int fit,
                             float *w, uint8_t *out)
{
    const int be = orc_block_elems(type);
    const size_t bb = orc_block_bytes(type);
    orc_row_weights_mode(x, q, n, sigma2, mode, w);
    /* A fitted unit (a legacy block or Q4_K sub-block of 32 weights, a Q6_K
     * sub-block of 16) whose importances are all zero -- an imatrix with no
     * data on those columns -- falls back to unit importances (reading). */
    const int unit = type == ORC_Q6_K ? 16 : 32;
    for (int64_t g = 0; g < n / unit; ++g) {
        int all_zero = 1;
        for (int i = 0; i < unit; ++i) if (w[unit * g + i] != 0.0f) { all_zero = 0; break; }
        if (all_zero) orc_row_weights_mode(x + unit * g, NULL, unit, sigma2, mode, w + unit * g);
    }
    for (int64_t ib = 0; ib < n / be; ++ib) {
        const float *xb = x + ib * be;
        float *wb = w + ib * be;
        if (type == ORC_Q4_K) quantize_kquant(xb, wb, fit, 15, out + ib * bb);
        else if (type == ORC_Q5_K) quantize_kquant(xb, wb, fit, 31, out + ib * bb);
        else if (type == ORC_Q6_K) quantize_q6k(xb, wb, out + ib * bb);
        else quantize_block32(type, xb, wb, out + ib * bb);
    }
    return ORC_OK;
}

static int weight_type_ok(int type)
{
    return type == ORC_Q4_0 || type == ORC_Q4_1 || type == ORC_Q5_0 ||
           type == ORC_Q5_1 || type == ORC_Q4_K || type == ORC_Q6_0 ||
           type == ORC_Q6_K || type == ORC_Q5_K;
}

int orc_quantize_row_sigma2_ex(int type, const float *x, const float *q,
                               int64_t n_per_row, float sigma2, int mode,
                               int fit, uint8_t *out)
{
    if (!weight_type_ok(type) || orc_row_bytes(type, n_per_row) == 0 ||
        mode < 0 || mode > ORC_W_IMATRIX_ONLY ||
        (fit != ORC_FIT_MAX && fit != ORC_FIT_WEIGHTED)) return ORC_EINVAL;
    float *w = (float *)malloc(sizeof(float) * (size_t)n_per_row);
    if (!w) return ORC_EINVAL;
    int rc = quantize_row_impl(type, x, q, n_per_row, sigma2, mode, fit, w, out);
    free(w);
    return rc;
}

int orc_quantize_row_sigma2_mode(int type, const float *x, const float *q,
                                 int64_t n_per_row, float sigma2, int mode,
                                 uint8_t *out)
{
    return orc_quantize_row_sigma2_ex(type, x, q, n_per_row, sigma2, mode,
                                      ORC_FIT_MAX, out);
}

int orc_quantize_row_sigma2(int type, const float *x, const float *q,
                            int64_t n_per_row, float sigma2, uint8_t *out)
{
    return orc_quantize_row_sigma2_mode(type, x, q, n_per_row, sigma2,
                                        ORC_W_SQRT_SIGMA2_X2, out);
}

static int quantize_rows_mode(int type, const float *x, const float *imatrix,
                              int64_t n_groups, int64_t rows_per_group,
                              int64_t n_per_row, int mode, int fit, uint8_t *out)
{
    if (!weight_type_ok(type) || n_groups < 0 || rows_per_group < 0 ||
        mode < 0 || mode > ORC_W_IMATRIX_ONLY ||
        (fit != ORC_FIT_MAX && fit != ORC_FIT_WEIGHTED)) return ORC_EINVAL;
    size_t rb = orc_row_bytes(type, n_per_row);
    if (rb == 0) return ORC_EINVAL;
    float *w = (float *)malloc(sizeof(float) * (size_t)n_per_row);
    if (!w) return ORC_EINVAL;
    for (int64_t r = 0; r < n_groups * rows_per_group; ++r) {
        const float *xr = x + r * n_per_row;
        const float *q = imatrix ? imatrix + (r / rows_per_group) * n_per_row : NULL;
        quantize_row_impl(type, xr, q, n_per_row, orc_row_sigma2(xr, n_per_row),
                          mode, fit, w, out + (size_t)r * rb);
    }
    free(w);
    return ORC_OK;
}

int orc_quantize_rows_grouped(int type, const float *x, const float *imatrix,
                              int64_t n_groups, int64_t rows_per_group,
                              int64_t n_per_row, uint8_t *out)
{
    return quantize_rows_mode(type, x, imatrix, n_groups, rows_per_group,
                              n_per_row, ORC_W_SQRT_SIGMA2_X2, ORC_FIT_MAX, out);
}

int orc_quantize_rows_ex(int type, const float *x, const float *imatrix,
                         int64_t n_groups, int64_t rows_per_group,
                         int64_t n_per_row, int mode, int fit, uint8_t *out)
{
    return quantize_rows_mode(type, x, imatrix, n_groups, rows_per_group,
                              n_per_row, mode, fit, out);
}

int orc_quantize_rows_weighted(int type, const float *x, const float *imatrix,
                               int64_t n_rows, int64_t n_per_row, int mode,
                               uint8_t *out)
{
    if (n_rows == 0) return weight_type_ok(type) && orc_row_bytes(type, n_per_row) ? ORC_OK : ORC_EINVAL;
    return quantize_rows_mode(type, x, imatrix, 1, n_rows, n_per_row, mode, ORC_FIT_MAX, out);
}

int orc_quantize_rows(int type, const float *x, const float *imatrix,
                      int64_t n_rows, int64_t n_per_row, uint8_t *out)
{
    if (n_rows == 0) return weight_type_ok(type) && orc_row_bytes(type, n_per_row) ? ORC_OK : ORC_EINVAL;
    return orc_quantize_rows_grouped(type, x, imatrix, 1, n_rows, n_per_row, out);
}

/* ------------------------------------------------------------------------ */
/* Q8_K_128 [Q8 §修复方案]                                                    */

/* One Q8_K block of B values (B = 128, 64 or 16): the scale, the codes,
 * then one int16 code sum per 32 codes (one per block when B = 16), then
 * zero bytes up to the block size. */
static void quantize_q8k_block(const float *xb, int B, size_t bb, uint8_t *o)
{
    float amax = 0.0f;
    for (int i = 0; i < B; ++i) amax = fmaxf(amax, fabsf(xb[i]));
    /* Readings: codes q = rint(x * 127/amax) in -127..127, scale
     * d = amax/127 stored as float, an all-zero block (or one whose
     * 127/amax is not finite) stores zeros. */
    float id = amax > 0.0f ? 127.0f / amax : 0.0f;
    int zero = !(amax > 0.0f) || !isfinite(id);
    float d = zero ? 0.0f : amax / 127.0f;
    int8_t q[128];
    for (int i = 0; i < B; ++i)
        q[i] = zero ? 0 : (int8_t)clampf(rintf(xb[i] * id), -127.0f, 127.0f);
    put_f32(o, d);
    memcpy(o + 4, q, (size_t)B);
    const int gs = B < 32 ? B : 32;
    for (int g = 0; g < B / gs; ++g) {
        int s = 0;
        for (int i = 0; i < gs; ++i) s += q[gs * g + i];
        int16_t s16 = (int16_t)s;   /* |s| <= 32*127 = 4064 */
        o[4 + B + 2 * g] = (uint8_t)(uint16_t)s16;
        o[5 + B + 2 * g] = (uint8_t)((uint16_t)s16 >> 8);
    }
    for (size_t k = 4 + (size_t)B + 2 * (size_t)(B / gs); k < bb; ++k)
        o[k] = 0;
}

int orc_quantize_q8k(int type, const float *x, int64_t n_rows,
                     int64_t n_per_row, uint8_t *out)
{
    if (type != ORC_Q8_K128 && type != ORC_Q8_K64 && type != ORC_Q8_K16)
        return ORC_EINVAL;
    size_t rb = orc_row_bytes(type, n_per_row);
    if (rb == 0 || n_rows < 0) return ORC_EINVAL;
    const int B = orc_block_elems(type);
    const size_t bb = orc_block_bytes(type);
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t ib = 0; ib < n_per_row / B; ++ib)
            quantize_q8k_block(x + r * n_per_row + ib * B, B, bb,
                               out + (size_t)r * rb + (size_t)ib * bb);
    return ORC_OK;
}

int orc_quantize_q8k128(const float *x, int64_t n_rows, int64_t n_per_row,
                        uint8_t *out)
{
    return orc_quantize_q8k(ORC_Q8_K128, x, n_rows, n_per_row, out);
}

/* ------------------------------------------------------------------------ */
/* decoders                                                                   */

static void unpack_nibbles32(const uint8_t *qs, uint8_t *u)
{
    for (int i = 0; i < 16; ++i) { u[i] = qs[i] & 15; u[i + 16] = qs[i] >> 4; }
}

int orc_dequantize_rows(int type, const uint8_t *in, int64_t n_rows,
                        int64_t n_per_row, float *out)
{
    size_t rb = orc_row_bytes(type, n_per_row);
    if (rb == 0 || n_rows < 0) return ORC_EINVAL;
    const int be = orc_block_elems(type);
    const size_t bb = orc_block_bytes(type);
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t ib = 0; ib < n_per_row / be; ++ib) {
            const uint8_t *p = in + (size_t)r * rb + (size_t)ib * bb;
            float *o = out + r * n_per_row + ib * be;
            uint8_t u[32];
            switch (type) {
            case ORC_Q4_0: case ORC_Q5_0: {
                int nmax = type == ORC_Q4_0 ? 8 : 16;
                float d = get_f32(p);
                if (type == ORC_Q4_0) {
                    unpack_nibbles32(p + 4, u);
                } else {
                    uint32_t qh = get_u32(p + 4);
                    unpack_nibbles32(p + 8, u);
                    for (int i = 0; i < 32; ++i) u[i] |= (uint8_t)(((qh >> i) & 1) << 4);
                }
                for (int i = 0; i < 32; ++i) o[i] = d * (float)((int)u[i] - nmax);
                break;
            }
            case ORC_Q4_1: case ORC_Q5_1: {
                float d = get_f32(p), m = get_f32(p + 4);
                if (type == ORC_Q4_1) {
                    unpack_nibbles32(p + 8, u);
                } else {
                    uint32_t qh = get_u32(p + 8);
                    unpack_nibbles32(p + 12, u);
                    for (int i = 0; i < 32; ++i) u[i] |= (uint8_t)(((qh >> i) & 1) << 4);
                }
                for (int i = 0; i < 32; ++i) o[i] = fmaf(d, (float)u[i], m);
                break;
            }
            case ORC_Q4_K: case ORC_Q5_K: {
                float dA = orc_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
                float dB = orc_f16_to_f32((uint16_t)(p[2] | (p[3] << 8)));
                uint8_t sc[8], mn[8];
                unpack6x8(p + 4, sc);
                unpack6x8(p + 10, mn);
                for (int j = 0; j < 8; ++j) {
                    float ds = dA * (float)sc[j], dm = dB * (float)mn[j];
                    if (type == ORC_Q4_K) {
                        unpack_nibbles32(p + 16 + 16 * j, u);
                    } else {
                        uint32_t qh = get_u32(p + 16 + 4 * j);
                        unpack_nibbles32(p + 48 + 16 * j, u);
                        for (int i = 0; i < 32; ++i) u[i] |= (uint8_t)(((qh >> i) & 1) << 4);
                    }
                    for (int i = 0; i < 32; ++i) o[32 * j + i] = fmaf(ds, (float)u[i], -dm);
                }
                break;
            }
            case ORC_Q8_K128: case ORC_Q8_K64: case ORC_Q8_K16: {
                float d = get_f32(p);
                for (int i = 0; i < be; ++i) o[i] = d * (float)(int8_t)p[4 + i];
                break;
            }
            case ORC_Q6_K: {
                float dA = orc_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
                for (int g = 0; g < 8; ++g) {
                    uint64_t plane = 0;
                    for (int k = 0; k < 8; ++k) plane |= (uint64_t)p[148 + 8 * g + k] << (8 * k);
                    unpack_nibbles32(p + 20 + 16 * g, u);
                    for (int i = 0; i < 32; ++i) {
                        int uu = u[i] | (int)(((plane >> (2 * i)) & 3) << 4);
                        float ds = dA * (float)(int8_t)p[4 + 2 * g + i / 16];
                        o[32 * g + i] = ds * (float)(uu - 32);
                    }
                }
                break;
            }
            case ORC_Q6_0: {
                float d = get_f32(p);
                uint64_t plane = 0;
                for (int k = 0; k < 8; ++k) plane |= (uint64_t)p[4 + k] << (8 * k);
                unpack_nibbles32(p + 12, u);
                for (int i = 0; i < 32; ++i) {
                    u[i] |= (uint8_t)(((plane >> (2 * i)) & 3) << 4);
                    o[i] = d * (float)((int)u[i] - 32);
                }
                break;
            }
            default:
                return ORC_EINVAL;
            }
        }
    }
    return ORC_OK;
}
