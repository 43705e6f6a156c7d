// imatrix.hip -- gfx950 kernels and C-ABI of the importance-matrix
// accumulator (declared in qrow_imatrix.h).
//
// Following these pages (cited by title and section):
//  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
//       的由来与原理", sections 一 and 六: per input column, the sum of squared
//       activations, per expert over the tokens routed to it.
//  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
//       i-quants", section 四: per-expert token counts beside the sums.
//
// Execution model. The work is a column reduction over tokens, bound by HBM
// reads of the activations, so the kernels are streaming kernels with no
// float atomics (the result must not depend on timing):
//  * k_imx_route (routed tensors only): turns the routing ids into a bitmap
//    [n_experts][n_tokens / 32]: bit t of expert e is set iff some slot of
//    token t names e. One workgroup per 64 tokens loads their ids at once,
//    builds its words for all experts in LDS (LDS atomic OR: order-free) and
//    writes them out, so a repeated expert within a token collapses to one
//    bit.
//  * k_imx_gather: one workgroup per (512-column chunk, expert, token slab).
//    Wave 0 expands the expert's bitmap words of a 4096-token window into an
//    ascending token list in LDS; the eight waves then take list entries
//    round-robin, each lane streaming 8 columns of a row per 16-byte load
//    (bf16), eight rows in flight, and accumulate a^2 in double. The
//    waves are combined in a fixed order. With one slab the workgroup owns
//    its (expert, chunk) cells and adds into the state directly; otherwise
//    it writes a partial that k_imx_reduce adds up in slab order.
//  * Slabs exist only to fill the chip when experts x chunks is small
//    (dense tensors, few experts): the host picks them from the shape.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qr_internal.h"
#include "qrow.h"
#include "qrow_imatrix.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int IMX_WAVES = 8;                     // waves per gather workgroup
constexpr int IMX_THREADS = WAVE * IMX_WAVES;
constexpr int IMX_LANE_COLS = 8;                 // columns per lane
constexpr int IMX_CHUNK = WAVE * IMX_LANE_COLS;  // columns per workgroup
constexpr int IMX_WIN_WORDS = 128;               // bitmap words per window
constexpr int IMX_WIN = IMX_WIN_WORDS * 32;      // tokens per window
constexpr int IMX_UNROLL = 8;                    // rows in flight per wave
constexpr int IMX_ROUTE_WORDS = 2;               // words per expert per route workgroup
constexpr int IMX_ROUTE_THREADS = 256;
constexpr int IMX_ROUTE_PER_THREAD = IMX_ROUTE_WORDS * 32 * QR_IMX_MAX_TOP_K / IMX_ROUTE_THREADS;
constexpr int IMX_TARGET_WGS = 256;              // gather workgroups wanted (8 waves each)
constexpr int IMX_MIN_SLAB_ROWS = 128;           // mean rows per (expert, slab), at least
constexpr int IMX_REDUCE_BATCH = 32;              // slab partials loaded at once
constexpr int IMX_RED_BYTES = (IMX_WAVES - 1) * IMX_CHUNK * 8;  // wave partials
constexpr int IMX_LDS_BYTES = IMX_RED_BYTES > IMX_WIN * 4 ? IMX_RED_BYTES : IMX_WIN * 4;

__host__ __device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// -------------------------------------------------------------------------
// routing bitmap [WT 六]

__global__ __launch_bounds__(IMX_ROUTE_THREADS) void k_imx_route(const int32_t* __restrict__ ids,
                                                                 int64_t n_tokens, int top_k, int n_experts,
                                                                 uint32_t* __restrict__ bitmap, int64_t n_words) {
  extern __shared__ uint32_t words[];  // [n_experts][IMX_ROUTE_WORDS]
  const int tid = threadIdx.x;
  const int n_cells = n_experts * IMX_ROUTE_WORDS;
  for (int i = tid; i < n_cells; i += IMX_ROUTE_THREADS) words[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * (IMX_ROUTE_WORDS * 32);
  const int64_t pairs_left = (n_tokens - t0) * top_k;
  const int n_pairs = (int)min64((int64_t)IMX_ROUTE_WORDS * 32 * top_k, pairs_left);
  const int32_t* ids_blk = ids + t0 * top_k;
  // all loads first (independent), then the LDS updates
  int v[IMX_ROUTE_PER_THREAD];
#pragma unroll
  for (int j = 0; j < IMX_ROUTE_PER_THREAD; ++j) {
    const int p = tid + j * IMX_ROUTE_THREADS;
    v[j] = p < n_pairs ? ids_blk[p] : -1;
  }
#pragma unroll
  for (int j = 0; j < IMX_ROUTE_PER_THREAD; ++j) {
    const int p = tid + j * IMX_ROUTE_THREADS;
    if ((unsigned)v[j] < (unsigned)n_experts) {
      const int lt = p / top_k;  // token within this workgroup's span
      atomicOr(&words[v[j] * IMX_ROUTE_WORDS + (lt >> 5)], 1u << (lt & 31));
    }
  }
  __syncthreads();
  const int64_t w0 = (int64_t)blockIdx.x * IMX_ROUTE_WORDS;
  for (int i = tid; i < n_cells; i += IMX_ROUTE_THREADS) {
    const int e = i / IMX_ROUTE_WORDS;
    const int w = i - e * IMX_ROUTE_WORDS;
    if (w0 + w < n_words) bitmap[(int64_t)e * n_words + w0 + w] = words[i];
  }
}

// -------------------------------------------------------------------------
// gather and accumulate [WT 一, 六] [LR 四]

__device__ __forceinline__ void add_sq(double (&acc)[IMX_LANE_COLS], const float (&v)[IMX_LANE_COLS]) {
#pragma unroll
  for (int k = 0; k < IMX_LANE_COLS; ++k) {
    const double d = (double)v[k];
    acc[k] = __builtin_fma(d, d, acc[k]);  // d*d is exact: one rounding, as d*d + acc
  }
}

// One lane's 8 columns of one row as loaded: 16 bytes of bf16 or 32 bytes
// of fp32 (the bf16 form uses the first vector only).
struct RawCols {
  u32x4 a, b;
};

template <bool BF16>
__device__ __forceinline__ RawCols load_cols(const void* __restrict__ act, int64_t elem, bool on) {
  RawCols r;
  r.a = u32x4{0u, 0u, 0u, 0u};
  r.b = u32x4{0u, 0u, 0u, 0u};
  if (on) {
    if (BF16) {
      r.a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(act) + elem);
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(act) + elem);
      r.a = p[0];
      r.b = p[1];
    }
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void add_raw(double (&acc)[IMX_LANE_COLS], const RawCols& r) {
  float v[IMX_LANE_COLS];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (BF16) {
      v[2 * k] = __builtin_bit_cast(float, r.a[k] << 16);
      v[2 * k + 1] = __builtin_bit_cast(float, r.a[k] & 0xFFFF0000u);
    } else {
      // copy the element out first: a bit cast of a vector-element lvalue
      // reads element 0 whatever the index
      const uint32_t lo = r.a[k], hi = r.b[k];
      v[k] = __builtin_bit_cast(float, lo);
      v[4 + k] = __builtin_bit_cast(float, hi);
    }
  }
  add_sq(acc, v);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(v, d, WAVE);
    if (lane >= d) v += o;
  }
  return v;
}

template <bool BF16, bool ROUTED, bool DIRECT>
__global__ __launch_bounds__(IMX_THREADS) void k_imx_gather(
    const void* __restrict__ act, int64_t n_tokens, int n_slots, int64_t n_cols, const int32_t* __restrict__ ids,
    int top_k, const uint32_t* __restrict__ bitmap, int64_t n_words, int64_t slab_tokens, int n_experts,
    double* __restrict__ sums, int64_t* __restrict__ counts, double* __restrict__ part,
    int32_t* __restrict__ part_counts) {
  // The token list (act row of each routed token, during the windows) and
  // the wave partials (after them) share one buffer.
  __shared__ double lds_buf[IMX_LDS_BYTES / 8];
  __shared__ int32_t list_len;
  int32_t* list = reinterpret_cast<int32_t*>(lds_buf);
  double(*red)[IMX_CHUNK] = reinterpret_cast<double(*)[IMX_CHUNK]>(lds_buf);

  const int chunk = blockIdx.x;
  const int e = blockIdx.y;
  const int slab = blockIdx.z;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int64_t col = (int64_t)chunk * IMX_CHUNK + lane * IMX_LANE_COLS;
  const bool active = col < n_cols;
  const int64_t t_begin = (int64_t)slab * slab_tokens;
  const int64_t t_end = min64(n_tokens, t_begin + slab_tokens);

  double acc[IMX_LANE_COLS];
#pragma unroll
  for (int k = 0; k < IMX_LANE_COLS; ++k) acc[k] = 0.0;
  int64_t matched = 0;

  for (int64_t w0 = t_begin; w0 < t_end; w0 += IMX_WIN) {
    int n;
    if (ROUTED) {
      // Wave 0 lists the window's tokens routed to e, in ascending order;
      // lane l expands bitmap words 2l and 2l+1 (slab starts are multiples
      // of 32 tokens, and bits past n_tokens are never set).
      if (wave == 0) {
        const int64_t word0 = w0 >> 5;
        const int64_t words_left = n_words - word0;
        uint32_t b0 = 0, b1 = 0;
        if (2 * lane < words_left && 2 * lane < IMX_WIN_WORDS)
          b0 = bitmap[(int64_t)e * n_words + word0 + 2 * lane];
        if (2 * lane + 1 < words_left && 2 * lane + 1 < IMX_WIN_WORDS)
          b1 = bitmap[(int64_t)e * n_words + word0 + 2 * lane + 1];
        // the window may run past the slab end: drop those tokens
        const int64_t lim = t_end - w0;  // tokens of this window inside the slab
        if (lim < IMX_WIN) {
          const int64_t base0 = 64 * lane, base1 = 64 * lane + 32;
          if (base0 >= lim) b0 = 0;
          else if (lim - base0 < 32) b0 &= (1u << (lim - base0)) - 1u;
          if (base1 >= lim) b1 = 0;
          else if (lim - base1 < 32) b1 &= (1u << (lim - base1)) - 1u;
        }
        const int cnt = __builtin_popcount(b0) + __builtin_popcount(b1);
        const int incl = wave_scan(cnt, lane);
        int pos = incl - cnt;
        const int64_t tb = w0 + 64 * lane;
        while (b0) {
          const int bit = __builtin_ctz(b0);
          b0 &= b0 - 1u;
          list[pos++] = (int32_t)((tb + bit) * n_slots);
        }
        while (b1) {
          const int bit = __builtin_ctz(b1);
          b1 &= b1 - 1u;
          list[pos++] = (int32_t)((tb + 32 + bit) * n_slots);
        }
        if (lane == WAVE - 1) list_len = incl;
      }
      __syncthreads();
      n = list_len;
      if (n_slots > 1) {
        // per-slot rows: the row of token t is that of its first slot naming
        // e (one exists: the bitmap bit came from one of its slots); eight
        // ids are loaded at a time
        for (int i = threadIdx.x; i < n; i += IMX_THREADS) {
          const int64_t t = list[i] / n_slots;
          const int32_t* r = ids + t * top_k;
          int found = -1;
          for (int s0 = 0; s0 < top_k && found < 0; s0 += 8) {
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = s0 + j < top_k ? r[s0 + j] : -1;
#pragma unroll
            for (int j = 7; j >= 0; --j)
              if (v[j] == e) found = s0 + j;
          }
          list[i] += found;
        }
        __syncthreads();
      }
    } else {
      n = (int)min64(IMX_WIN, t_end - w0);
    }
    matched += n;

    // Entries wave, wave + W, wave + 2W, ... (W waves) in ascending order
    // per lane, U rows in flight (128 bytes per lane).
    constexpr int U = BF16 ? IMX_UNROLL : IMX_UNROLL / 2;
    for (int base = wave; base < n; base += IMX_WAVES * U) {
      RawCols r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * IMX_WAVES;
        const bool ok = i < n;  // uniform across the wave
        const int64_t row = ROUTED ? (int64_t)list[ok ? i : 0] : w0 + (ok ? i : 0);
        r[u] = load_cols<BF16>(act, row * n_cols + col, ok && active);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + u * IMX_WAVES < n) add_raw<BF16>(acc, r[u]);
    }
    if (ROUTED) __syncthreads();  // the list is rebuilt for the next window
  }

  // Combine the waves in the fixed order (((w0 + w1) + w2) + ...) + w7. The
  // partials overwrite the token list: the barrier that ends every routed
  // window orders its last reads before these writes.
  if (wave > 0) {
#pragma unroll
    for (int k = 0; k < IMX_LANE_COLS; ++k) red[wave - 1][lane * IMX_LANE_COLS + k] = acc[k];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < IMX_WAVES - 1; ++w)
#pragma unroll
    for (int k = 0; k < IMX_LANE_COLS; ++k) acc[k] += red[w][lane * IMX_LANE_COLS + k];
  if (active) {
    const int64_t cell = (int64_t)e * n_cols + col;
    if (DIRECT) {
#pragma unroll
      for (int k = 0; k < IMX_LANE_COLS; ++k) sums[cell + k] += acc[k];
    } else {
      double* p = part + (int64_t)slab * n_experts * n_cols + cell;
#pragma unroll
      for (int k = 0; k < IMX_LANE_COLS; ++k) p[k] = acc[k];
    }
  }
  if (chunk == 0 && lane == 0) {
    if (DIRECT)
      counts[e] += matched;
    else
      part_counts[(int64_t)slab * n_experts + e] = (int32_t)matched;
  }
}

// Adds the slab partials into the state, in slab order.
__global__ __launch_bounds__(64) void k_imx_reduce(const double* __restrict__ part,
                                                    const int32_t* __restrict__ part_counts, int n_slabs,
                                                    int64_t n_cells, int n_experts, double* __restrict__ sums,
                                                    int64_t* __restrict__ counts) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_cells; i += stride) {
    double s = 0.0;  // (0 + p0) + p1 ...: the sums are non-negative
    for (int k0 = 0; k0 < n_slabs; k0 += IMX_REDUCE_BATCH) {
      double v[IMX_REDUCE_BATCH];  // one batch of loads in flight
#pragma unroll
      for (int j = 0; j < IMX_REDUCE_BATCH; ++j)
        v[j] = k0 + j < n_slabs ? part[(int64_t)(k0 + j) * n_cells + i] : 0.0;
#pragma unroll
      for (int j = 0; j < IMX_REDUCE_BATCH; ++j) s += v[j];
    }
    sums[i] += s;
  }
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < n_experts; e += blockDim.x) {
      int64_t c = 0;
      for (int k = 0; k < n_slabs; ++k) c += part_counts[(int64_t)k * n_experts + e];
      counts[e] += c;
    }
  }
}

// -------------------------------------------------------------------------
// merge and finalize [LR 四]

__global__ __launch_bounds__(256) void k_imx_merge(double* __restrict__ sums, int64_t* __restrict__ counts,
                                                   const double* __restrict__ src_sums,
                                                   const int64_t* __restrict__ src_counts, int64_t n_cells,
                                                   int64_t n_experts) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_cells; i += stride)
    sums[i] += src_sums[i];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_experts; i += stride)
    counts[i] += src_counts[i];
}

__global__ __launch_bounds__(256) void k_imx_finalize(const double* __restrict__ sums,
                                                      const int64_t* __restrict__ counts, int64_t n_cols,
                                                      int64_t n_cells, float* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_cells; i += stride) {
    const int64_t c = counts[i / n_cols];
    q[i] = c > 0 ? (float)(sums[i] / (double)c) : 0.0f;
  }
}

// -------------------------------------------------------------------------
// host side

struct ImxPlan {
  int64_t chunks = 0, slabs = 0, slab_tokens = 0, n_words = 0;
  size_t bitmap_bytes = 0, part_bytes = 0, part_counts_bytes = 0, total = 0;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Launch plan for a valid shape (n_tokens > 0).
ImxPlan imx_plan(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n_cols) {
  ImxPlan p;
  p.chunks = (n_cols + IMX_CHUNK - 1) / IMX_CHUNK;
  p.slabs = 1;
  const int64_t base = p.chunks * n_experts;
  if (base < IMX_TARGET_WGS) {
    const int64_t want = (IMX_TARGET_WGS + base - 1) / base;
    const int64_t rows = n_tokens * (top_k > 0 ? top_k : 1);
    int64_t cap = rows / (n_experts * IMX_MIN_SLAB_ROWS);
    if (cap < 1) cap = 1;
    p.slabs = want < cap ? want : cap;
  }
  int64_t st = (n_tokens + p.slabs - 1) / p.slabs;
  st = (st + 31) & ~(int64_t)31;
  p.slab_tokens = st;
  p.slabs = (n_tokens + st - 1) / st;
  p.n_words = (n_tokens + 31) / 32;
  p.bitmap_bytes = top_k > 0 ? align256((size_t)n_experts * (size_t)p.n_words * 4) : 0;
  if (p.slabs > 1) {
    p.part_bytes = align256((size_t)p.slabs * (size_t)n_experts * (size_t)n_cols * 8);
    p.part_counts_bytes = align256((size_t)p.slabs * (size_t)n_experts * 4);
  }
  p.total = p.bitmap_bytes + p.part_bytes + p.part_counts_bytes;
  return p;
}

int validate_shape(int64_t n_tokens, int64_t n_slots, int64_t n_cols, bool routed, int64_t top_k,
                   int64_t n_experts) {
  if (n_tokens < 0 || top_k < 0) return qr_fail(QR_EINVAL_SHAPE, "negative n_tokens or top_k");
  if (n_cols <= 0 || n_cols % 8 != 0)
    return qr_fail(QR_EINVAL_SHAPE, "n_cols=%lld must be a positive multiple of 8", (long long)n_cols);
  if (n_experts < 1 || n_experts > QR_IMX_MAX_EXPERTS)
    return qr_fail(QR_EINVAL_SHAPE, "n_experts=%lld must be in [1, %d]", (long long)n_experts, QR_IMX_MAX_EXPERTS);
  if (!routed) {
    if (n_experts != 1 || n_slots != 1)
      return qr_fail(QR_EINVAL_SHAPE, "a dense tensor (top_k 0) needs n_experts 1 and n_slots 1");
  } else {
    if (top_k < 1 || top_k > QR_IMX_MAX_TOP_K)
      return qr_fail(QR_EINVAL_SHAPE, "top_k=%lld must be in [1, %d]", (long long)top_k, QR_IMX_MAX_TOP_K);
    if (n_slots != 1 && n_slots != top_k)
      return qr_fail(QR_EINVAL_SHAPE, "n_slots=%lld must be 1 or top_k", (long long)n_slots);
  }
  if (n_tokens > (int64_t)INT32_MAX / n_slots) return qr_fail(QR_EOVERFLOW, "n_tokens * n_slots >= 2^31");
  if (n_cols > INT64_MAX / 8 / n_experts || n_tokens * n_slots > INT64_MAX / 4 / n_cols)
    return qr_fail(QR_EOVERFLOW, "size overflows");
  return QR_OK;
}

template <bool BF16, bool ROUTED, bool DIRECT>
void launch_gather(dim3 grid, hipStream_t s, const void* act, int64_t n_tokens, int n_slots, int64_t n_cols,
                   const int32_t* ids, int top_k, const uint32_t* bitmap, int64_t n_words, int64_t slab_tokens,
                   int n_experts, double* sums, int64_t* counts, double* part, int32_t* part_counts) {
  hipLaunchKernelGGL((k_imx_gather<BF16, ROUTED, DIRECT>), grid, dim3(IMX_THREADS), 0, s, act, n_tokens, n_slots,
                     n_cols, ids, top_k, bitmap, n_words, slab_tokens, n_experts, sums, counts, part, part_counts);
}

template <bool BF16>
void dispatch_gather(bool routed, bool direct, dim3 grid, hipStream_t s, const void* act, int64_t n_tokens,
                     int n_slots, int64_t n_cols, const int32_t* ids, int top_k, const uint32_t* bitmap,
                     int64_t n_words, int64_t slab_tokens, int n_experts, double* sums, int64_t* counts,
                     double* part, int32_t* part_counts) {
#define QR_IMX_LAUNCH(R, D)                                                                                     \
  launch_gather<BF16, R, D>(grid, s, act, n_tokens, n_slots, n_cols, ids, top_k, bitmap, n_words, slab_tokens, \
                            n_experts, sums, counts, part, part_counts)
  if (routed) {
    if (direct) QR_IMX_LAUNCH(true, true);
    else QR_IMX_LAUNCH(true, false);
  } else {
    if (direct) QR_IMX_LAUNCH(false, true);
    else QR_IMX_LAUNCH(false, false);
  }
#undef QR_IMX_LAUNCH
}

int elementwise_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

extern "C" {

size_t qr_imatrix_workspace_bytes(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n_cols) {
  const int64_t n_slots = 1;
  if (n_tokens <= 0) return 0;
  int rc = validate_shape(n_tokens, n_slots, n_cols, top_k > 0, top_k, n_experts);
  if (rc != QR_OK) return 0;
  return imx_plan(n_tokens, top_k, n_experts, n_cols).total;
}

int qr_imatrix_accumulate(int src, const void* act, int64_t n_tokens, int64_t n_slots, int64_t n_cols,
                          const int32_t* ids, int64_t top_k, int64_t n_experts, double* sums, int64_t* counts,
                          void* workspace, size_t workspace_bytes, void* stream) {
  qr_clear_error();
  if (src != QR_F32 && src != QR_BF16) return qr_fail(QR_EINVAL_TYPE, "source dtype %d is not f32/bf16", src);
  const bool routed = top_k != 0;
  int rc = validate_shape(n_tokens, n_slots, n_cols, routed, top_k, n_experts);
  if (rc != QR_OK) return rc;
  if (n_tokens == 0) return QR_OK;
  if (!act || !sums || !counts) return qr_fail(QR_EINVAL_PTR, "act, sums and counts must be non-NULL");
  if (routed && !ids) return qr_fail(QR_EINVAL_PTR, "top_k > 0 needs the routing ids");
  if (!qr_aligned(act, 16) || !qr_aligned(sums, 16) || !qr_aligned(counts, 8) || !qr_aligned(ids, 4))
    return qr_fail(QR_EINVAL_PTR, "act and sums must be 16-byte, counts 8-byte and ids 4-byte aligned");
  const ImxPlan p = imx_plan(n_tokens, top_k, n_experts, n_cols);
  if (p.total > 0) {
    if (!workspace) return qr_fail(QR_EINVAL_PTR, "this shape needs a workspace of %zu bytes", p.total);
    if (workspace_bytes < p.total)
      return qr_fail(QR_EINVAL_SHAPE, "workspace_bytes=%zu < %zu needed", workspace_bytes, p.total);
    if (!qr_aligned(workspace, 256)) return qr_fail(QR_EINVAL_PTR, "workspace must be 256-byte aligned");
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint32_t* bitmap = routed ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  double* part = p.slabs > 1 ? reinterpret_cast<double*>(ws + p.bitmap_bytes) : nullptr;
  int32_t* part_counts = p.slabs > 1 ? reinterpret_cast<int32_t*>(ws + p.bitmap_bytes + p.part_bytes) : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  if (routed) {
    const int64_t route_grid = (p.n_words + IMX_ROUTE_WORDS - 1) / IMX_ROUTE_WORDS;
    const size_t lds = (size_t)n_experts * IMX_ROUTE_WORDS * 4;
    hipLaunchKernelGGL(k_imx_route, dim3((uint32_t)route_grid), dim3(IMX_ROUTE_THREADS), lds, s, ids, n_tokens,
                       (int)top_k, (int)n_experts, bitmap, p.n_words);
    rc = qr_check_launch("k_imx_route");
    if (rc != QR_OK) return rc;
  }
  const bool direct = p.slabs == 1;
  const dim3 grid((uint32_t)p.chunks, (uint32_t)n_experts, (uint32_t)p.slabs);
  if (src == QR_BF16)
    dispatch_gather<true>(routed, direct, grid, s, act, n_tokens, (int)n_slots, n_cols, ids, (int)top_k, bitmap,
                          p.n_words, p.slab_tokens, (int)n_experts, sums, counts, part, part_counts);
  else
    dispatch_gather<false>(routed, direct, grid, s, act, n_tokens, (int)n_slots, n_cols, ids, (int)top_k, bitmap,
                           p.n_words, p.slab_tokens, (int)n_experts, sums, counts, part, part_counts);
  rc = qr_check_launch("k_imx_gather");
  if (rc != QR_OK || direct) return rc;
  const int64_t n_cells = n_experts * n_cols;
  int64_t rgrid = (n_cells + 63) / 64;
  if (rgrid > 8192) rgrid = 8192;
  hipLaunchKernelGGL(k_imx_reduce, dim3((uint32_t)rgrid), dim3(64), 0, s, part, part_counts, (int)p.slabs,
                     n_cells, (int)n_experts, sums, counts);
  return qr_check_launch("k_imx_reduce");
}

int qr_imatrix_merge(double* sums, int64_t* counts, const double* src_sums, const int64_t* src_counts,
                     int64_t n_experts, int64_t n_cols, void* stream) {
  qr_clear_error();
  if (n_experts < 0 || n_cols < 0) return qr_fail(QR_EINVAL_SHAPE, "negative size");
  if (n_experts == 0 || n_cols == 0) return QR_OK;
  if (n_cols > INT64_MAX / 8 / n_experts) return qr_fail(QR_EOVERFLOW, "size overflows");
  if (!sums || !counts || !src_sums || !src_counts) return qr_fail(QR_EINVAL_PTR, "NULL state pointer");
  if (!qr_aligned(sums, 8) || !qr_aligned(src_sums, 8) || !qr_aligned(counts, 8) || !qr_aligned(src_counts, 8))
    return qr_fail(QR_EINVAL_PTR, "state pointers must be 8-byte aligned");
  const int64_t n_cells = n_experts * n_cols;
  hipLaunchKernelGGL(k_imx_merge, dim3(elementwise_grid(n_cells)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     sums, counts, src_sums, src_counts, n_cells, n_experts);
  return qr_check_launch("k_imx_merge");
}

int qr_imatrix_finalize(const double* sums, const int64_t* counts, int64_t n_experts, int64_t n_cols, float* q,
                        void* stream) {
  qr_clear_error();
  if (n_experts < 0 || n_cols < 0) return qr_fail(QR_EINVAL_SHAPE, "negative size");
  if (n_experts == 0 || n_cols == 0) return QR_OK;
  if (n_cols > INT64_MAX / 8 / n_experts) return qr_fail(QR_EOVERFLOW, "size overflows");
  if (!sums || !counts || !q) return qr_fail(QR_EINVAL_PTR, "NULL pointer");
  if (!qr_aligned(sums, 8) || !qr_aligned(counts, 8) || !qr_aligned(q, 4))
    return qr_fail(QR_EINVAL_PTR, "misaligned pointer");
  const int64_t n_cells = n_experts * n_cols;
  hipLaunchKernelGGL(k_imx_finalize, dim3(elementwise_grid(n_cells)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), sums, counts, n_cols, n_cells, q);
  return qr_check_launch("k_imx_finalize");
}

}  // extern "C"
