/*
 * qrow_imatrix.h -- C-ABI of libqrow.so, part 2: the importance-matrix
 * accumulator, which produces the per-column importances (imatrix) that the
 * row quantizers of qrow.h consume.
 *
 * The operations follow these pages (cited by title and section):
 *  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
 *       的由来与原理", section 一: the importance of a weight is a diagonal
 *       Hessian estimate, one value per input column of the tensor; section
 *       六: for a stacked expert tensor the squared input activations are
 *       accumulated per expert, only over the tokens routed to that expert,
 *       so an expert that is never routed has no data.
 *  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
 *       i-quants", section 四: each expert keeps its own activation (token)
 *       count beside its full sums; with counts by token, merging two
 *       collections is correct and independent of the batch size.
 *
 * Accumulator state (caller-owned device memory, zero-filled for a fresh
 * accumulator):
 *   sums   double  [n_experts, n_cols]   sum of a^2 per expert and column
 *   counts int64_t [n_experts]           tokens accumulated per expert
 * A dense tensor is the case n_experts == 1 without routing ids. The
 * importance is q[e][c] = sums[e][c] / counts[e] (qr_imatrix_finalize).
 *
 * Conventions are those of qrow.h: device pointers, asynchronous calls on
 * `stream`, return 0 or a negative QR_E* code with nothing launched on
 * failure and a message in qr_last_error(). The library allocates nothing:
 * scratch memory is passed in as `workspace`.
 *
 * Numerics: a^2 of an fp32 or bf16 value is exact in double, so the only
 * rounding is in the additions. The kernels add in a fixed order that
 * depends only on the shapes (never on timing), so results are
 * reproducible bit for bit; against a sequential double sum in token order
 * each sum differs by at most (n + 1) * 2^-53 of its value, n being the
 * number of tokens added.
 */
#ifndef QROW_IMATRIX_H
#define QROW_IMATRIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QR_IMX_MAX_EXPERTS 1024   /* experts per stacked tensor */
#define QR_IMX_MAX_TOP_K   64     /* routed slots per token     */

/*
 * qr_imatrix_workspace_bytes -- bytes of device scratch memory that
 * qr_imatrix_accumulate needs for this shape (0 if none; then workspace may
 * be NULL). top_k is 0 for a dense tensor. Returns 0 for invalid shapes too;
 * the accumulate call reports those.
 */
size_t qr_imatrix_workspace_bytes(int64_t n_tokens, int64_t top_k,
                                  int64_t n_experts, int64_t n_cols);

/*
 * qr_imatrix_accumulate -- adds one batch of activations to the state
 * [WT 一, 六] [LR 四].
 *  src      QR_F32 or QR_BF16 (enum of qrow.h): element type of act.
 *  act      [n_tokens, n_slots, n_cols], 16-byte aligned. n_slots == 1: one
 *           row per token, seen by every expert the token is routed to;
 *           n_slots == top_k: one row per routed slot, slot s of token t
 *           seen by expert ids[t][s] only.
 *  ids, top_k  int32 [n_tokens, top_k] expert ids with top_k >= 1; or
 *           top_k == 0 for a dense tensor (ids unused, may be NULL; then
 *           n_experts == 1, n_slots == 1 and every token counts). An id
 *           outside [0, n_experts) marks an unused slot and is skipped; an
 *           expert named twice by one token counts once, with the row of the
 *           first such slot.
 *  sums, counts  the state, updated in place: for every (token, expert)
 *           routing, sums[e][c] += a[c]^2 for all c and counts[e] += 1.
 *  workspace, workspace_bytes  device scratch of at least
 *           qr_imatrix_workspace_bytes(...) bytes, 256-byte aligned; its
 *           contents on entry do not matter and are clobbered.
 * Limits: n_cols a positive multiple of 8; 1 <= n_experts <= 1024;
 * 0 <= top_k <= 64; n_tokens * n_slots < 2^31. n_tokens == 0 is a no-op. Calls that share a state or a workspace must be ordered on one
 * stream (or synchronized by the caller).
 */
int qr_imatrix_accumulate(int src, const void *act, int64_t n_tokens,
                          int64_t n_slots, int64_t n_cols, const int32_t *ids,
                          int64_t top_k, int64_t n_experts, double *sums,
                          int64_t *counts, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * qr_imatrix_merge -- adds another state (src_sums, src_counts), e.g. a
 * collection over other text, into (sums, counts) [LR 四]. Element-wise
 * double and integer additions.
 */
int qr_imatrix_merge(double *sums, int64_t *counts, const double *src_sums,
                     const int64_t *src_counts, int64_t n_experts,
                     int64_t n_cols, void *stream);

/*
 * qr_imatrix_finalize -- q[e][c] = sums[e][c] / counts[e] divided in double
 * and rounded once to float; 0 for an expert with counts[e] == 0 (no data:
 * the caller decides, from counts, whether the tensor is covered). q is fp32
 * [n_experts, n_cols]; row e is the imatrix argument of qr_quantize_rows
 * (or row e of qr_quantize_rows_grouped's) for expert e.
 */
int qr_imatrix_finalize(const double *sums, const int64_t *counts,
                        int64_t n_experts, int64_t n_cols, float *q,
                        void *stream);

#ifdef __cplusplus
}
#endif
#endif
