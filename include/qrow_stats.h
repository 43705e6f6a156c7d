/*
 * qrow_stats.h -- C-ABI of libqrow.so, part 4: error statistics of packed
 * rows against the rows they were quantized from (a quantize-stats report).
 *
 * The statistics follow these pages (cited by title and section):
 *  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
 *       i-quants", section 3.2: the quantize-stats tool reports the RMSE,
 *       sqrt(total error / number of samples), the maximum error and the
 *       95th percentile of the error.
 *  [WT] "ik_llama.cpp 量化权重之谜 …", section 一: the importance-weighted
 *       squared error that the quantizer minimizes.
 *
 * Conventions are those of qrow.h (device pointers, 16-byte aligned;
 * asynchronous calls on `stream`; 0 or a negative QR_E* code with nothing
 * launched on failure; the library allocates nothing: scratch memory is the
 * caller's `workspace`).
 */
#ifndef QROW_STATS_H
#define QROW_STATS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Written by qr_quantize_stats (device memory, 72 bytes). With e_i = x_i -
 * xhat_i in float (xhat from qr_dequantize_rows) and q_i the imatrix entry
 * of the element's column (1 without an imatrix): */
typedef struct {
    double sum_err2;     /* sum e_i^2                                       */
    double sum_x2;       /* sum x_i^2                                       */
    double sum_werr2;    /* sum q_i e_i^2                                   */
    double sum_wx2;      /* sum q_i x_i^2                                   */
    float max_abs_err;   /* max |e_i|                                       */
    float p95_abs_err;   /* the ceil(0.95 N)-th smallest |e_i| (exact)      */
    int64_t n;           /* N = n_rows * n_per_row                          */
    double rmse;         /* sqrt(sum_err2 / N)                              */
    double rel_rmse;     /* sqrt(sum_err2 / sum_x2), 0 if sum_x2 is 0       */
    double weighted_rel_rmse; /* sqrt(sum_werr2 / sum_wx2), 0 if that is 0  */
} qr_stats;

/* Device scratch bytes that qr_quantize_stats needs (a few hundred KB; 0
 * for invalid shapes). */
size_t qr_stats_workspace_bytes(int64_t n_rows, int64_t n_per_row);

/*
 * qr_quantize_stats -- error statistics of `packed` (type t, any qr_type,
 * [n_rows, qr_row_bytes(t, n_per_row)]) against `x` (src fp32 or bf16,
 * [n_rows, n_per_row]), weighted by `imatrix` ([n_per_row] fp32 or NULL).
 * RMSE = sqrt(sum_err2 / n); relative RMSE = sqrt(sum_err2 / sum_x2);
 * importance-weighted relative RMSE = sqrt(sum_werr2 / sum_wx2), all three
 * computed on the device in double from the sums. max and
 * p95 are exact (the percentile by a radix selection over the bits of |e|,
 * in three counting passes); the sums are double, added in a fixed order
 * (reproducible bit for bit), each within n * 2^-52 of its exact value,
 * relative. Limits: n_rows * n_per_row < 2^32; n_per_row a multiple of 32
 * (for Q8_K16: an even number of blocks). Calls that share `out` or the
 * workspace must be ordered on one stream.
 */
int qr_quantize_stats(int t, int src, const void *x, const void *packed,
                      const float *imatrix, int64_t n_rows, int64_t n_per_row,
                      qr_stats *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Size of the device workspace that qr_quantize_stats_noalloc keeps in a
 * static array, one per GPU (the same as qr_stats_workspace_bytes). */
#define QR_STATS_STATIC_SCRATCH_BYTES 377088

/*
 * qr_quantize_stats_noalloc -- qr_quantize_stats for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments and results (bit for bit)
 * as qr_quantize_stats, without the workspace: the library keeps it in a
 * static device array of QR_STATS_STATIC_SCRATCH_BYTES per GPU, which
 * covers every call that qr_quantize_stats accepts (n_rows * n_per_row
 * below 2^32; larger calls return QR_EOVERFLOW before any launch). The
 * array's device address is looked up once per device, on the first call
 * whose stream belongs to it; nothing is allocated, then or later. Every
 * call clears what must start at zero with a kernel (no memset). All calls
 * on one GPU share that GPU's array: calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race
 * and give undefined results; order them on one stream.
 */
int qr_quantize_stats_noalloc(int t, int src, const void *x, const void *packed,
                              const float *imatrix, int64_t n_rows,
                              int64_t n_per_row, qr_stats *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif
