/*
 * imatrix_oracle.c -- CPU oracle for the importance-matrix accumulator.
 *
 * TEST INFRASTRUCTURE ONLY (see qrow_oracle.c for the rules that apply to
 * the whole oracle): a plain, slow, single-threaded definition that the GPU
 * library is checked against, sharing no code with it.
 *
 * Sources, cited by page title and section:
 *  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
 *       的由来与原理". Section 一: the importance qw of a weight is the
 *       diagonal Hessian estimate that the imatrix tool computes, one value
 *       per element of the weight row, i.e. one per input column. Section 六:
 *       for a stacked expert tensor the collector reads the routing ids and
 *       adds the squared input activations only to the experts that a token
 *       was actually routed to, so an expert that is never routed has no
 *       statistics.
 *  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
 *       i-quants", section 四 (4.1, 4.2): every expert of a stacked tensor
 *       keeps its own activation count next to its full sums, which is what
 *       makes merging two collections correct; counting tokens (activations)
 *       rather than chunks makes the result independent of the batch size.
 *
 * Readings (the pages fix the quantities, not the arithmetic):
 *  - the accumulated quantity per (expert, column) is the sum of a^2 over the
 *    tokens routed to the expert, and the count is the number of such
 *    tokens; the importance handed to the quantizer is their ratio, the mean
 *    of a^2;
 *  - sums are kept in double: a^2 of a float is exact in double, so the only
 *    rounding is in the additions, taken here in ascending token order (and
 *    ascending slot order within a token);
 *  - a routing id outside [0, n_experts) marks an unused slot and is skipped;
 *    a token routed twice to one expert counts once, with the activation of
 *    the first such slot;
 *  - with one activation row per token (n_slots == 1) every routed expert
 *    sees that row; with one row per slot (n_slots == top_k) the expert of
 *    slot s sees row s;
 *  - the importance of an expert with no tokens is reported as 0 (its count
 *    of 0 tells the caller that the data are missing).
 */
#include "orc_qrow.h"

int orc_imatrix_accumulate(const float *act, int64_t n_tokens, int64_t n_slots,
                           int64_t n_cols, const int32_t *ids, int64_t top_k,
                           int64_t n_experts, double *sums, int64_t *counts)
{
    if (n_tokens < 0 || n_cols <= 0 || n_experts <= 0)
        return ORC_EINVAL;
    if (ids == NULL) {
        if (n_experts != 1 || n_slots != 1)
            return ORC_EINVAL;
    } else if (top_k <= 0 || (n_slots != 1 && n_slots != top_k)) {
        return ORC_EINVAL;
    }
    const int64_t n_route = ids ? top_k : 1;
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int64_t s = 0; s < n_route; ++s) {
            int64_t e = 0;
            if (ids) {
                e = ids[t * top_k + s];
                if (e < 0 || e >= n_experts)
                    continue;                       /* unused slot */
                int seen = 0;
                for (int64_t s2 = 0; s2 < s; ++s2)
                    if (ids[t * top_k + s2] == e)
                        seen = 1;
                if (seen)
                    continue;                       /* already counted */
            }
            const int64_t row = t * n_slots + (n_slots == 1 ? 0 : s);
            const float *a = act + row * n_cols;
            double *acc = sums + e * n_cols;
            for (int64_t c = 0; c < n_cols; ++c)
                acc[c] += (double)a[c] * (double)a[c];
            counts[e] += 1;
        }
    }
    return ORC_OK;
}

int orc_imatrix_merge(double *sums, int64_t *counts, const double *src_sums,
                      const int64_t *src_counts, int64_t n_experts,
                      int64_t n_cols)
{
    if (n_experts < 0 || n_cols < 0)
        return ORC_EINVAL;
    for (int64_t e = 0; e < n_experts; ++e) {
        for (int64_t c = 0; c < n_cols; ++c)
            sums[e * n_cols + c] += src_sums[e * n_cols + c];
        counts[e] += src_counts[e];
    }
    return ORC_OK;
}

int orc_imatrix_finalize(const double *sums, const int64_t *counts,
                         int64_t n_experts, int64_t n_cols, float *q)
{
    if (n_experts < 0 || n_cols < 0)
        return ORC_EINVAL;
    for (int64_t e = 0; e < n_experts; ++e)
        for (int64_t c = 0; c < n_cols; ++c)
            q[e * n_cols + c] = counts[e] > 0
                ? (float)(sums[e * n_cols + c] / (double)counts[e])
                : 0.0f;
    return ORC_OK;
}
