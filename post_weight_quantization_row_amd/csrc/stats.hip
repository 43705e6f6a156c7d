// stats.hip -- gfx950 kernels and C-ABI of the quantization error statistics
// (declared in qrow_stats.h).
//
// Following these pages (cited by title and section):
//  [LR] "量化方法论实证：为什么 LQER/L²QER 难以改进 ik_llama.cpp 的 k-quants 与
//       i-quants", section 3.2: RMSE, maximum error and 95th percentile of a
//       quantized tensor against the original.
//  [WT] "ik_llama.cpp 量化权重之谜 …", section 一: the importance-weighted
//       squared error.
//
// Execution model. Each 32-element group is handled by eight lanes (four
// elements each, 16-byte loads of x): the lanes decode their elements from
// the packed block with the format's decoder arithmetic, form e = x - xhat
// in float and take |e|. Three passes over the tensor select the exact
// nearest-rank 95th percentile by the bits of |e| (non-negative floats order
// like their bit patterns): pass 0 also accumulates the double sums and the
// maximum and counts the top 11 bits in per-workgroup LDS histograms; passes
// 1 and 2 count the next 11 and the last 9 bits among the elements whose
// leading bits match the prefix selected so far. Counting is integer
// (order-free) and the sums are combined in a fixed order, so results are
// reproducible bit for bit. One-wave kernels between the passes pick the
// histogram bin that holds the wanted rank.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "qr_internal.h"
#include "qrow.h"
#include "qrow_stats.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int ST_THREADS = 256;
constexpr int ST_LANES = 8;                               // lanes per 32-element group
constexpr int ST_GROUPS_PER_WG = ST_THREADS / ST_LANES;   // 32
constexpr int ST_MAX_WGS = 2048;
constexpr int ST_BINS0 = 2048, ST_BINS1 = 2048, ST_BINS2 = 512;  // bits 30..20, 19..9, 8..0
constexpr int ST_PART = 5;                                // doubles per workgroup partial

struct StatsState {
  uint32_t k;       // rank (1-based) still to find within the selected prefix
  uint32_t prefix;  // leading bits of the value selected so far
};

// The global histograms are kept in ST_REP copies, workgroup b adding into
// copy b % ST_REP, so that thousands of workgroups do not queue on the same
// few counters; the select kernels add the copies up.
constexpr int ST_REP = 16;

// workspace layout
constexpr size_t WS_STATE = 0;
constexpr size_t WS_HIST0 = 256;
constexpr size_t WS_HIST1 = WS_HIST0 + (size_t)ST_REP * ST_BINS0 * 4;
constexpr size_t WS_HIST2 = WS_HIST1 + (size_t)ST_REP * ST_BINS1 * 4;
constexpr size_t WS_PART = (WS_HIST2 + (size_t)ST_REP * ST_BINS2 * 4 + 255) & ~(size_t)255;
constexpr size_t WS_BYTES = WS_PART + (size_t)ST_MAX_WGS * ST_PART * 8;

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ float f32_bits(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ float half_bits(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// Decoded values of elements 4k .. 4k+3 of 32-element group gin of a packed
// row, with the decoders' arithmetic (qr_dequantize_rows).
template <int TYPE>
__device__ __forceinline__ void decode4(const uint8_t* __restrict__ row, int gin, int k, float (&xh)[4]) {
  if (TYPE == QR_Q8_K128 || TYPE == QR_Q8_K64 || TYPE == QR_Q8_K16) {
    // block of values 32*gin + 4k .. +3 and the offset of their code word
    const uint8_t* b = TYPE == QR_Q8_K128 ? row + (int64_t)(gin >> 2) * 140
                     : TYPE == QR_Q8_K64  ? row + (int64_t)(gin >> 1) * 72
                                          : row + (int64_t)(2 * gin + (k >> 2)) * 24;
    const int off = TYPE == QR_Q8_K128 ? 4 + 32 * (gin & 3) + 4 * k
                  : TYPE == QR_Q8_K64  ? 4 + 32 * (gin & 1) + 4 * k
                                       : 4 + 4 * (k & 3);
    const float d = f32_bits(ld32(b));
    const uint32_t w = ld32(b + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) xh[e] = d * (float)(int8_t)(uint8_t)(w >> (8 * e));
  } else if (TYPE == QR_Q4_K || TYPE == QR_Q5_K) {
    constexpr bool Q5 = TYPE == QR_Q5_K;
    const uint8_t* sb = row + (int64_t)(gin >> 3) * (Q5 ? 176 : 144);
    const int j = gin & 7;
    const uint32_t h0 = ld32(sb), h1 = ld32(sb + 4), h2 = ld32(sb + 8), h3 = ld32(sb + 12);
    const uint64_t sc6 = (uint64_t)h1 | ((uint64_t)(h2 & 0xffffu) << 32);
    const uint64_t mn6 = (uint64_t)(h2 >> 16) | ((uint64_t)h3 << 16);
    const float ds = half_bits(h0) * (float)((sc6 >> (6 * j)) & 63);
    const float dm = half_bits(h0 >> 16) * (float)((mn6 >> (6 * j)) & 63);
    const uint32_t w = ld32(sb + (Q5 ? 48 : 16) + 16 * j + 4 * (k & 3));
    const uint32_t nib = k < 4 ? (w & 0x0f0f0f0fu) : ((w >> 4) & 0x0f0f0f0fu);
    const uint32_t qh = Q5 ? ld32(sb + 16 + 4 * j) >> (4 * k) : 0u;   // fifth bits of elements 4k ..
#pragma unroll
    for (int e = 0; e < 4; ++e)
      xh[e] = __builtin_fmaf(ds, (float)(((nib >> (8 * e)) & 0xffu) | (((qh >> e) & 1u) << 4)), -dm);
  } else if (TYPE == QR_Q6_K) {
    const uint8_t* p = row + (int64_t)(gin >> 3) * 212;
    const int j = gin & 7;
    const float dA = half_bits(ld32(p));
    const uint32_t sw = ld32(p + 4 + 4 * (j >> 1));
    const float ds = dA * (float)(int)(int8_t)(uint8_t)(sw >> (8 * (2 * (j & 1) + (k >> 2))));
    const uint32_t qh = ld32(p + 148 + 8 * j + 4 * (k >> 2));
    const uint32_t w = ld32(p + 20 + 16 * j + 4 * (k & 3));
    const uint32_t nib = k < 4 ? (w & 0x0f0f0f0fu) : ((w >> 4) & 0x0f0f0f0fu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = ((nib >> (8 * e)) & 0xffu) | (((qh >> (2 * (4 * (k & 3) + e))) & 3u) << 4);
      xh[e] = ds * (float)((int)u - 32);
    }
  } else if (TYPE == QR_Q6_0) {
    const uint8_t* p = row + (int64_t)gin * 28;
    const float d = f32_bits(ld32(p));
    const uint32_t qh = ld32(p + 4 + 4 * (k >> 2));   // the plane of elements 16*(k/4) ..
    const uint32_t w = ld32(p + 12 + 4 * (k & 3));
    const uint32_t nib = k < 4 ? (w & 0x0f0f0f0fu) : ((w >> 4) & 0x0f0f0f0fu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = ((nib >> (8 * e)) & 0xffu) | (((qh >> (2 * (4 * (k & 3) + e))) & 3u) << 4);
      xh[e] = d * (float)((int)u - 32);
    }
  } else {
    constexpr bool SYM = TYPE == QR_Q4_0 || TYPE == QR_Q5_0;
    constexpr bool FIVE = TYPE == QR_Q5_0 || TYPE == QR_Q5_1;
    constexpr int BYTES = TYPE == QR_Q4_0 ? 20 : TYPE == QR_Q5_1 ? 28 : 24;
    const uint8_t* p = row + (int64_t)gin * BYTES;
    const float d = f32_bits(ld32(p));
    const float m = SYM ? 0.0f : f32_bits(ld32(p + 4));
    const uint32_t qh = FIVE ? ld32(p + (SYM ? 4 : 8)) : 0u;
    const uint8_t* qs = p + (TYPE == QR_Q4_0 ? 4 : TYPE == QR_Q5_1 ? 12 : 8);
    const uint32_t w = ld32(qs + 4 * (k & 3));
    const uint32_t nib = k < 4 ? (w & 0x0f0f0f0fu) : ((w >> 4) & 0x0f0f0f0fu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t u = (nib >> (8 * e)) & 0xffu;
      if (FIVE) u |= ((qh >> (4 * k + e)) & 1u) << 4;
      if (SYM) xh[e] = d * (float)((int)u - (FIVE ? 16 : 8));
      else xh[e] = __builtin_fmaf(d, (float)u, m);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void load_x4(const void* __restrict__ x, int64_t elem, float (&v)[4]) {
  if (BF16) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(x) + elem);
    const uint32_t a = r[0], b = r[1];
    v[0] = f32_bits(a << 16);
    v[1] = f32_bits(a & 0xffff0000u);
    v[2] = f32_bits(b << 16);
    v[3] = f32_bits(b & 0xffff0000u);
  } else {
    const f32x4 r = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + elem);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = r[e];
  }
}

// One workgroup per histogram copy clears it; the first sets the state.
__global__ __launch_bounds__(ST_THREADS) void k_stats_init(uint8_t* __restrict__ ws, uint32_t k) {
  const int r = blockIdx.x;
  uint32_t* h0 = reinterpret_cast<uint32_t*>(ws + WS_HIST0) + r * ST_BINS0;
  uint32_t* h1 = reinterpret_cast<uint32_t*>(ws + WS_HIST1) + r * ST_BINS1;
  uint32_t* h2 = reinterpret_cast<uint32_t*>(ws + WS_HIST2) + r * ST_BINS2;
  for (int i = threadIdx.x; i < ST_BINS0; i += ST_THREADS) h0[i] = 0;
  for (int i = threadIdx.x; i < ST_BINS1; i += ST_THREADS) h1[i] = 0;
  for (int i = threadIdx.x; i < ST_BINS2; i += ST_THREADS) h2[i] = 0;
  if (r == 0 && threadIdx.x == 0) {
    StatsState* st = reinterpret_cast<StatsState*>(ws + WS_STATE);
    st->k = k;
    st->prefix = 0;
  }
}

template <int TYPE, bool BF16, int PASS>
__global__ __launch_bounds__(ST_THREADS) void k_stats_pass(const void* __restrict__ x, const uint8_t* __restrict__ packed,
                                                           const float* __restrict__ q, int64_t n_groups,
                                                           int groups_per_row, int n_per_row, int64_t row_bytes,
                                                           uint8_t* __restrict__ ws) {
  constexpr int NB = PASS == 2 ? ST_BINS2 : ST_BINS0;
  __shared__ uint32_t h[NB];
  __shared__ double red[ST_THREADS / WAVE][ST_PART];
  for (int i = threadIdx.x; i < NB; i += ST_THREADS) h[i] = 0;
  __syncthreads();
  const uint32_t prefix = PASS > 0 ? reinterpret_cast<const StatsState*>(ws + WS_STATE)->prefix : 0u;
  const int k = threadIdx.x & (ST_LANES - 1);
  double s_e2 = 0.0, s_x2 = 0.0, s_qe2 = 0.0, s_qx2 = 0.0;
  float mx = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * ST_GROUPS_PER_WG;
  for (int64_t gg = (int64_t)blockIdx.x * ST_GROUPS_PER_WG + threadIdx.x / ST_LANES; gg < n_groups; gg += stride) {
    const int64_t r = gg / groups_per_row;
    const int gin = (int)(gg - r * groups_per_row);
    float xh[4], xv[4];
    decode4<TYPE>(packed + r * row_bytes, gin, k, xh);
    load_x4<BF16>(x, r * n_per_row + gin * 32 + 4 * k, xv);
    float qv[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if (PASS == 0 && q) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(q + gin * 32 + 4 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = t[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float err = xv[e] - xh[e];
      const float ae = fabsf(err);
      const uint32_t bits = __builtin_bit_cast(uint32_t, ae);
      if (PASS == 0) {
        const double ed = (double)err, xd = (double)xv[e], qd = (double)qv[e];
        const double e2 = ed * ed, x2 = xd * xd;  // squares of floats: exact in double
        s_e2 += e2;                               // one rounding per term
        s_x2 += x2;
        s_qe2 = __builtin_fma(qd, e2, s_qe2);     // one rounding per term
        s_qx2 = __builtin_fma(qd, x2, s_qx2);
        mx = fmaxf(mx, ae);
        atomicAdd(&h[bits >> 20], 1u);
      } else if (PASS == 1) {
        if ((bits >> 20) == prefix) atomicAdd(&h[(bits >> 9) & 2047u], 1u);
      } else {
        if ((bits >> 9) == prefix) atomicAdd(&h[bits & 511u], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = reinterpret_cast<uint32_t*>(ws + (PASS == 0 ? WS_HIST0 : PASS == 1 ? WS_HIST1 : WS_HIST2)) +
                 (blockIdx.x % ST_REP) * NB;
  for (int i = threadIdx.x; i < NB; i += ST_THREADS)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  if (PASS != 0) return;
  // sums: butterfly over the wave, then the waves in order
  double v[ST_PART] = {s_e2, s_x2, s_qe2, s_qx2, (double)mx};
#pragma unroll
  for (int m = WAVE / 2; m >= 1; m >>= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] += __shfl_xor(v[c], m, WAVE);
    v[4] = fmax(v[4], __shfl_xor(v[4], m, WAVE));
  }
  const int wave = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) {
#pragma unroll
    for (int c = 0; c < ST_PART; ++c) red[wave][c] = v[c];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* part = reinterpret_cast<double*>(ws + WS_PART) + (int64_t)blockIdx.x * ST_PART;
    double a[ST_PART] = {red[0][0], red[0][1], red[0][2], red[0][3], red[0][4]};
    for (int w = 1; w < ST_THREADS / WAVE; ++w) {
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] += red[w][c];
      a[4] = fmax(a[4], red[w][4]);
    }
#pragma unroll
    for (int c = 0; c < ST_PART; ++c) part[c] = a[c];
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, WAVE);
    if (lane >= d) v += o;
  }
  return v;
}

// One workgroup: the bin of the histogram (the sum of its copies) that
// holds rank k; appends its index (BITS bits) to the prefix and leaves the
// rank within the bin.
template <int NB, int BITS, int PASS>
__global__ __launch_bounds__(ST_THREADS) void k_stats_select(uint8_t* __restrict__ ws) {
  constexpr int PER = NB / ST_THREADS;
  __shared__ uint32_t wave_tot[ST_THREADS / WAVE];
  const uint32_t* h = reinterpret_cast<const uint32_t*>(ws + (PASS == 0 ? WS_HIST0 : PASS == 1 ? WS_HIST1 : WS_HIST2));
  StatsState* st = reinterpret_cast<StatsState*>(ws + WS_STATE);
  const int t = threadIdx.x, lane = t & (WAVE - 1), wave = t / WAVE;
  uint32_t c[PER];
  uint32_t local = 0;
#pragma unroll
  for (int b = 0; b < PER; ++b) {
    uint32_t v = 0;
#pragma unroll
    for (int r = 0; r < ST_REP; ++r) v += h[r * NB + t * PER + b];
    c[b] = v;
    local += v;
  }
  uint32_t incl = wave_scan(local, lane);
  if (lane == WAVE - 1) wave_tot[wave] = incl;
  const uint32_t k = st->k;
  __syncthreads();  // the wave totals are in place and every thread has read k
  for (int w = 0; w < wave; ++w) incl += wave_tot[w];
  const uint32_t excl = incl - local;
  if (excl < k && k <= incl) {
    uint32_t cum = excl;
    int bin = t * PER + PER - 1;
    uint32_t rem = k - cum;
#pragma unroll
    for (int b = 0; b < PER; ++b) {
      if (cum + c[b] >= k) {
        bin = t * PER + b;
        rem = k - cum;
        break;
      }
      cum += c[b];
    }
    st->prefix = (st->prefix << BITS) | (uint32_t)bin;
    st->k = rem;
  }
}

// Sums of the per-workgroup partials in a fixed order (thread t takes
// partials t, t + 256, ..., then a tree over the threads), then the output.
__global__ __launch_bounds__(ST_THREADS) void k_stats_final(const uint8_t* __restrict__ ws, int n_wgs, int64_t n,
                                                            qr_stats* __restrict__ out) {
  __shared__ double red[ST_PART][ST_THREADS];
  const double* part = reinterpret_cast<const double*>(ws + WS_PART);
  const int t = threadIdx.x;
  double v[ST_PART] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int w = t; w < n_wgs; w += ST_THREADS) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] += part[(int64_t)w * ST_PART + c];
    v[4] = fmax(v[4], part[(int64_t)w * ST_PART + 4]);
  }
#pragma unroll
  for (int c = 0; c < ST_PART; ++c) red[c][t] = v[c];
  __syncthreads();
  for (int m = ST_THREADS / 2; m >= 1; m >>= 1) {
    if (t < m) {
#pragma unroll
      for (int c = 0; c < 4; ++c) red[c][t] += red[c][t + m];
      red[4][t] = fmax(red[4][t], red[4][t + m]);
    }
    __syncthreads();
  }
  if (t == 0) {
    const StatsState* st = reinterpret_cast<const StatsState*>(ws + WS_STATE);
    out->sum_err2 = red[0][0];
    out->sum_x2 = red[1][0];
    out->sum_werr2 = red[2][0];
    out->sum_wx2 = red[3][0];
    out->max_abs_err = (float)red[4][0];
    out->p95_abs_err = __builtin_bit_cast(float, st->prefix);
    out->n = n;
    out->rmse = sqrt(red[0][0] / (double)n);
    out->rel_rmse = red[1][0] > 0.0 ? sqrt(red[0][0] / red[1][0]) : 0.0;
    out->weighted_rel_rmse = red[3][0] > 0.0 ? sqrt(red[2][0] / red[3][0]) : 0.0;
  }
}

template <int TYPE, bool BF16>
int run_stats(const void* x, const uint8_t* packed, const float* q, int64_t n_rows, int n_per_row, int64_t rb,
              qr_stats* out, uint8_t* ws, hipStream_t s) {
  const int64_t n = n_rows * n_per_row;
  const int64_t n_groups = n / 32;
  int64_t grid = (n_groups + ST_GROUPS_PER_WG - 1) / ST_GROUPS_PER_WG;
  if (grid > ST_MAX_WGS) grid = ST_MAX_WGS;
  const uint32_t k = (uint32_t)((95 * n + 99) / 100);
  const int gpr = n_per_row / 32;
  hipLaunchKernelGGL(k_stats_init, dim3(ST_REP), dim3(ST_THREADS), 0, s, ws, k);
  hipLaunchKernelGGL((k_stats_pass<TYPE, BF16, 0>), dim3((uint32_t)grid), dim3(ST_THREADS), 0, s, x, packed, q,
                     n_groups, gpr, n_per_row, rb, ws);
  hipLaunchKernelGGL((k_stats_select<ST_BINS0, 11, 0>), dim3(1), dim3(ST_THREADS), 0, s, ws);
  hipLaunchKernelGGL((k_stats_pass<TYPE, BF16, 1>), dim3((uint32_t)grid), dim3(ST_THREADS), 0, s, x, packed, q,
                     n_groups, gpr, n_per_row, rb, ws);
  hipLaunchKernelGGL((k_stats_select<ST_BINS1, 11, 1>), dim3(1), dim3(ST_THREADS), 0, s, ws);
  hipLaunchKernelGGL((k_stats_pass<TYPE, BF16, 2>), dim3((uint32_t)grid), dim3(ST_THREADS), 0, s, x, packed, q,
                     n_groups, gpr, n_per_row, rb, ws);
  hipLaunchKernelGGL((k_stats_select<ST_BINS2, 9, 2>), dim3(1), dim3(ST_THREADS), 0, s, ws);
  hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(ST_THREADS), 0, s, ws, (int)grid, n, out);
  return qr_check_launch("k_stats");
}

template <bool BF16>
int dispatch_stats(int t, const void* x, const uint8_t* packed, const float* q, int64_t n_rows, int n_per_row,
                   int64_t rb, qr_stats* out, uint8_t* ws, hipStream_t s) {
  switch (t) {
    case QR_Q4_0: return run_stats<QR_Q4_0, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q4_1: return run_stats<QR_Q4_1, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q5_0: return run_stats<QR_Q5_0, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q5_1: return run_stats<QR_Q5_1, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q4_K: return run_stats<QR_Q4_K, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q6_0: return run_stats<QR_Q6_0, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q8_K64: return run_stats<QR_Q8_K64, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q8_K16: return run_stats<QR_Q8_K16, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q6_K: return run_stats<QR_Q6_K, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    case QR_Q5_K: return run_stats<QR_Q5_K, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
    default: return run_stats<QR_Q8_K128, BF16>(x, packed, q, n_rows, n_per_row, rb, out, ws, s);
  }
}

}  // namespace

// The allocation-free entry point's workspace: one copy per GPU (each device
// that loads the library holds it until the process ends). Host code never
// uses this name as an address: it takes each device's address of the array
// from hipGetSymbolAddress, with that device current, once per device.
static_assert(WS_BYTES == QR_STATS_STATIC_SCRATCH_BYTES, "the header states the static workspace's size");
static __device__ __align__(256) uint8_t scratch[WS_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch[SCRATCH_MAX_DEVICES];   // device address of `scratch` on each device, once resolved

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream), resolved on the first call for that device.
int scratch_for(hipStream_t stream, uint8_t** ws) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return qr_fail(QR_EDEVICE, "hipGetDevice failed");
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipStreamGetDevice failed");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return qr_fail(QR_EDEVICE, "device %d beyond the library's table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipSetDevice(%d) failed", dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return qr_fail(QR_EDEVICE, "hipSetDevice(%d) failed", cur);
    if (e != hipSuccess || !p) return qr_fail(QR_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ws = reinterpret_cast<uint8_t*>(g_scratch[dev]);
  return QR_OK;
}

// Argument checks shared by both entry points; 1 means "nothing to do".
int stats_check(int t, int src, const void* x, const void* packed, const float* imatrix, int64_t n_rows,
                int64_t n_per_row, const qr_stats* out) {
  if (t < QR_Q4_0 || t > QR_Q5_K) return qr_fail(QR_EINVAL_TYPE, "unknown type %d", t);
  if (src != QR_F32 && src != QR_BF16) return qr_fail(QR_EINVAL_TYPE, "source dtype %d is not f32/bf16", src);
  const size_t rb = qr_row_bytes(t, n_per_row);
  if (n_rows < 0 || n_per_row <= 0 || rb == 0 || n_per_row % 32 != 0)
    return qr_fail(QR_EINVAL_SHAPE, "n_per_row=%lld is not a positive multiple of the block length and of 32",
                   (long long)n_per_row);
  if (n_rows == 0) return 1;
  if (n_per_row > INT32_MAX || n_rows > (int64_t)UINT32_MAX / n_per_row)
    return qr_fail(QR_EOVERFLOW, "n_rows * n_per_row must be below 2^32");
  if (!x || !packed || !out) return qr_fail(QR_EINVAL_PTR, "x, packed and out must be non-NULL");
  if (!qr_aligned(x, 16) || !qr_aligned(packed, 16) || (imatrix && !qr_aligned(imatrix, 16)) || !qr_aligned(out, 8))
    return qr_fail(QR_EINVAL_PTR, "misaligned pointer (x, packed, imatrix: 16; out: 8)");
  return QR_OK;
}

int stats_launch(int t, int src, const void* x, const void* packed, const float* imatrix, int64_t n_rows,
                 int64_t n_per_row, qr_stats* out, uint8_t* ws, hipStream_t s) {
  const int64_t rb = (int64_t)qr_row_bytes(t, n_per_row);
  const uint8_t* p = reinterpret_cast<const uint8_t*>(packed);
  return src == QR_F32 ? dispatch_stats<false>(t, x, p, imatrix, n_rows, (int)n_per_row, rb, out, ws, s)
                       : dispatch_stats<true>(t, x, p, imatrix, n_rows, (int)n_per_row, rb, out, ws, s);
}

}  // namespace

extern "C" {

size_t qr_stats_workspace_bytes(int64_t n_rows, int64_t n_per_row) {
  if (n_rows < 0 || n_per_row <= 0) return 0;
  return WS_BYTES;
}

int qr_quantize_stats_noalloc(int t, int src, const void* x, const void* packed, const float* imatrix,
                              int64_t n_rows, int64_t n_per_row, qr_stats* out, void* stream) {
  qr_clear_error();
  const int rc = stats_check(t, src, x, packed, imatrix, n_rows, n_per_row, out);
  if (rc != QR_OK) return rc < 0 ? rc : QR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  const int rs = scratch_for(s, &ws);
  if (rs != QR_OK) return rs;
  return stats_launch(t, src, x, packed, imatrix, n_rows, n_per_row, out, ws, s);
}

int qr_quantize_stats(int t, int src, const void* x, const void* packed, const float* imatrix, int64_t n_rows,
                      int64_t n_per_row, qr_stats* out, void* workspace, size_t workspace_bytes, void* stream) {
  qr_clear_error();
  const int rc = stats_check(t, src, x, packed, imatrix, n_rows, n_per_row, out);
  if (rc != QR_OK) return rc < 0 ? rc : QR_OK;
  if (!workspace) return qr_fail(QR_EINVAL_PTR, "workspace must be non-NULL");
  if (!qr_aligned(workspace, 256)) return qr_fail(QR_EINVAL_PTR, "misaligned workspace (256 bytes)");
  if (workspace_bytes < WS_BYTES) return qr_fail(QR_EINVAL_SHAPE, "workspace_bytes=%zu < %zu", workspace_bytes, WS_BYTES);
  return stats_launch(t, src, x, packed, imatrix, n_rows, n_per_row, out, reinterpret_cast<uint8_t*>(workspace),
                      reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
