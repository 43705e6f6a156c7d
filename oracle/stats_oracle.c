/*
 * stats_oracle.c -- CPU oracle for the quantization error statistics (test
 * infrastructure only; see qrow_oracle.c for the rules of the oracle).
 *
 * Sources, cited by page title and section:
 *  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
 *       i-quants", section 3.2: the quantize-stats tool reports the RMSE as
 *       sqrt(total error / number of samples), the maximum error and the 95th
 *       percentile of the error.
 *  [WT] "ik_llama.cpp 量化权重之谜 …", section 一: the importance-weighted
 *       squared error the quantizer minimizes.
 *
 * Readings: the error of element i is e_i = x_i - xhat_i, one float
 * subtraction, with xhat_i the value the format's decoder gives
 * (orc_dequantize_rows); the 95th percentile is the nearest-rank one, the
 * k-th smallest |e_i| with k = ceil(0.95 N); the sums are in double, in
 * element order: sum e^2, sum x^2, sum q e^2 and sum q x^2 (q the imatrix
 * entry of the element's column, 1 without an imatrix). From the sums:
 * RMSE = sqrt(sum e^2 / N), relative RMSE = sqrt(sum e^2 / sum x^2) and the
 * importance-weighted relative RMSE = sqrt(sum q e^2 / sum q x^2).
 */
#include "orc_qrow.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int cmp_float(const void *a, const void *b)
{
    const float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

int orc_quantize_stats(int type, const float *x, const uint8_t *packed,
                       const float *q, int64_t n_rows, int64_t n_per_row,
                       double *sums, float *max_abs, float *p95_abs)
{
    if (n_rows <= 0 || orc_row_bytes(type, n_per_row) == 0 || n_per_row <= 0)
        return ORC_EINVAL;
    const int64_t n = n_rows * n_per_row;
    float *xh = malloc(sizeof(float) * (size_t)n);
    float *ae = malloc(sizeof(float) * (size_t)n);
    if (!xh || !ae) {
        free(xh); free(ae);
        return ORC_EINVAL;
    }
    orc_dequantize_rows(type, packed, n_rows, n_per_row, xh);
    double e2 = 0.0, x2 = 0.0, qe2 = 0.0, qx2 = 0.0;
    float mx = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float e = x[i] - xh[i];
        const double qi = q ? (double)q[i % n_per_row] : 1.0;
        const double ed = (double)e, xd = (double)x[i];
        e2 += ed * ed;
        x2 += xd * xd;
        qe2 += qi * (ed * ed);
        qx2 += qi * (xd * xd);
        ae[i] = fabsf(e);
        mx = fmaxf(mx, ae[i]);
    }
    qsort(ae, (size_t)n, sizeof(float), cmp_float);
    const int64_t k = (95 * n + 99) / 100;      /* ceil(0.95 n), 1-based */
    sums[0] = e2;
    sums[1] = x2;
    sums[2] = qe2;
    sums[3] = qx2;
    /* [LR 3.2]: RMSE = sqrt(total error / number of samples); the relative
     * forms divide by the signal instead (0 when that is 0). */
    sums[4] = sqrt(e2 / (double)n);
    sums[5] = x2 > 0.0 ? sqrt(e2 / x2) : 0.0;
    sums[6] = qx2 > 0.0 ? sqrt(qe2 / qx2) : 0.0;
    *max_abs = mx;
    *p95_abs = ae[k - 1];
    free(xh);
    free(ae);
    return ORC_OK;
}
