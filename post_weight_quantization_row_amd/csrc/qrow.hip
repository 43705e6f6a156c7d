// qrow.hip -- gfx950 kernels and the C-ABI of libqrow.so.
//
// Importance-matrix-weighted row quantization, following these pages (cited
// by title and section):
//  [WT] "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
//       的由来与原理", section 一: row statistic sigma2, element importance
//       qw*sqrt(sigma2 + x^2), least-squares block scale sumlx/suml2 and
//       greedy level flips along g = scale*w*(x - scale*l).
//  [KQ] "3.2 K-quants 与重要性矩阵：量化兵器谱", section 一: Q4_K super-block
//       (Q5_K: the same super-block with 5-bit levels; the layout is ours).
//  [LQ] "从零理解 LLM 量化 PTQ、QAT 与 ik_llama.cpp 量化体系的源码级导学", 2.1:
//       legacy 32-weight blocks.
//  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …", 修复方案:
//       Q8_K_128 activation blocks.
//
// Execution model (gfx950, wave64):
//  * Weight rows: one workgroup per row, of one wave per 64 groups of 32
//    weights (at most eight waves; a width whose groups leave lanes of the
//    last wave idle walks blocks of consecutive rows instead, see
//    k_quantize_rows_stream). The workgroup streams the row from HBM
//    once with coalesced 16-byte loads into LDS (32-element groups padded to
//    a 16-byte multiple so that per-lane group reads are bank-conflict free)
//    while accumulating sum x^2 in double; a workgroup reduction gives
//    sigma2. Each lane then owns one 32-element group at a
//    time and solves it entirely in VGPRs: importances, trial scales,
//    least-squares sums, the sequential flip passes (sequential within a
//    lane, parallel across the 64 lanes), packing. For the K types, eight
//    consecutive lanes hold the eight 32-weight parts of one super-block and
//    combine their scales with cross-lane shuffles.
//  * Activations (Q8_K_128) and the decoders are streaming kernels: 32 lanes
//    per 128-value block (one float4 each), several blocks in flight per
//    wave.
//
// Numerics: every float operation that decides a code is written out
// explicitly (fmaf where fused, no contraction: built with
// -ffp-contract=off), divisions and square roots are correctly rounded, and
// sums run in ascending element order inside one lane, so the outputs are
// bit-identical to a sequential single-precision evaluation of the same
// steps. The row sum of x^2 is accumulated in double; only the order of its
// additions differs from a sequential sum, which can move sigma2 by one ulp
// when the double sum lies within a few units of its last place of a float
// rounding boundary.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>

#include "qrow.h"
#include "qr_internal.h"

namespace {

// native vector types (usable with the nontemporal builtins)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int QK = 32;                  // weights per fitted group
constexpr int LDS_F32_STRIDE = 36;      // floats per staged group (32 + pad)
constexpr int LDS_BF16_STRIDE = 40;     // bf16 per staged group (32 + pad)

// Solver constants: trial-scale spacing and counts, flip passes.
constexpr float CAND_STEP = 0.25f;
constexpr int SYM_CAND = 5;
constexpr int SYM_FLIP_PASSES = 1;
constexpr int ASYM_CAND = 3;
constexpr int ASYM_FLIP_PASSES = 1;

// Trial k uses (nmax + CAND_STEP * offset(k)): 0, -1, +1, -2, +2.
__host__ __device__ constexpr int cand_offset(int k) {
  return k == 0 ? 0 : ((k & 1) ? -((k + 1) / 2) : k / 2);
}

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ float rne(float v) { return __builtin_rintf(v); }
__device__ __forceinline__ float med3(float v, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(v, lo, hi);
}
__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }

// The same value, opaque to the optimizer (no instruction is emitted): an
// expression formed again from it is computed afresh instead of being kept
// live, as a 32-wide array of registers, from its first evaluation.
__device__ __forceinline__ float fresh(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Correctly rounded square root for t in [2^-96, FLT_MAX]: the hardware
// square root s (within one ulp) is corrected to the nearest float by
// Tuckerman's test, exact with fused multiply-adds. The sign of the exact
// residual t - s*s says on which side of sqrt(t) s lies, so only the
// neighbour n on the other side can be nearer: n replaces s iff
// t - n*s > 0 (n above s) or t - n*s <= 0 (n below s). Outside that range
// the library sqrtf is used.
__device__ __forceinline__ float sqrt_cr(float t, bool normal_range) {
  if (!normal_range) return sqrtf(t);
  const float s = __builtin_amdgcn_sqrtf(t);
  const bool up = fma_(-s, s, t) > 0.0f;   // s < sqrt(t)
  const float n = __builtin_bit_cast(float, __builtin_bit_cast(int32_t, s) + (up ? 1 : -1));
  const bool pos = fma_(-n, s, t) > 0.0f;
  return pos == up ? n : s;
}

// -------------------------------------------------------------------------
// DPP helpers (gfx9 encodings): quad_perm, row_half_mirror, row_mirror, row_shl:8
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_SHL8 = 0x108;

// max and bitwise or over each group of 8 lanes (8s .. 8s+7): two quad
// swaps, then the mirror within the half row joins the two quads
__device__ __forceinline__ float oct_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  return fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
}
__device__ __forceinline__ uint32_t oct_or(uint32_t v) {
  v |= (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)v);
  v |= (uint32_t)dpp_i<DPP_QUAD_XOR2>((int)v);
  return v | (uint32_t)dpp_i<DPP_ROW_HALF_MIRROR>((int)v);
}

// -------------------------------------------------------------------------
// row staging and the row statistic [WT 一]

// The workgroup streams its row into LDS (16-byte coalesced loads; groups of
// 32 padded to a 16-byte multiple) and returns this wave's sum of x^2 in
// double, reduced across the wave.
template <bool BF16>
__device__ __forceinline__ double stage_row(const void* __restrict__ xrow, int n, void* lds, int tid, int nthreads) {
  // Thread tid moves 16-byte vectors tid, tid + nthreads, ... As nthreads is
  // a multiple of 64, each step advances the vector by nthreads/8 (fp32) or
  // nthreads/4 (bf16) whole groups and keeps its place inside the group, so
  // both addresses advance by a fixed stride.
  double acc = 0.0;
  if (!BF16) {
    const int n4 = n >> 2;
    const f32x4* src = reinterpret_cast<const f32x4*>(xrow) + tid;
    float* dst = reinterpret_cast<float*>(lds) + (tid >> 3) * LDS_F32_STRIDE + (tid & 7) * 4;
    const int dstep = (nthreads >> 3) * LDS_F32_STRIDE;
#pragma unroll 8
    for (int i = tid; i < n4; i += nthreads) {
      f32x4 v = __builtin_nontemporal_load(src);
      *reinterpret_cast<f32x4*>(dst) = v;
      src += nthreads;
      dst += dstep;
      acc = __builtin_fma((double)v.x, (double)v.x, acc);
      acc = __builtin_fma((double)v.y, (double)v.y, acc);
      acc = __builtin_fma((double)v.z, (double)v.z, acc);
      acc = __builtin_fma((double)v.w, (double)v.w, acc);
    }
  } else {
    const int n8 = n >> 3;
    const u32x4* src = reinterpret_cast<const u32x4*>(xrow) + tid;
    uint16_t* dst = reinterpret_cast<uint16_t*>(lds) + (tid >> 2) * LDS_BF16_STRIDE + (tid & 3) * 8;
    const int dstep = (nthreads >> 2) * LDS_BF16_STRIDE;
#pragma unroll 8
    for (int i = tid; i < n8; i += nthreads) {
      u32x4 v = __builtin_nontemporal_load(src);
      *reinterpret_cast<u32x4*>(dst) = v;
      src += nthreads;
      dst += dstep;
      const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double a = (double)__builtin_bit_cast(float, p[k] << 16);
        const double b = (double)__builtin_bit_cast(float, p[k] & 0xffff0000u);
        acc = __builtin_fma(a, a, acc);
        acc = __builtin_fma(b, b, acc);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, WAVE);
  return acc;
}

// The same staging in two steps, for the streaming kernel: stage_row_load
// fetches this thread's vectors of the row into registers, and
// stage_row_store writes them to LDS and returns the wave's sum of x^2, in the
// order stage_row takes it. A row of at most 64 W groups gives each of the
// 64 W threads at most 4 vectors (bf16) or 8 (fp32).
template <bool BF16>
struct RowRegs {
  static constexpr int N = BF16 ? 4 : 8;
  u32x4 v[N];
};

template <bool BF16>
__device__ __forceinline__ void stage_row_load(const void* __restrict__ xrow, int n, int tid, int nthreads,
                                               RowRegs<BF16>& rr) {
  const int nv = BF16 ? n >> 3 : n >> 2;
  const u32x4* src = reinterpret_cast<const u32x4*>(xrow);
#pragma unroll
  for (int k = 0; k < RowRegs<BF16>::N; ++k) {
    const int i = tid + k * nthreads;
    rr.v[k] = u32x4{0u, 0u, 0u, 0u};
    if (i < nv) rr.v[k] = __builtin_nontemporal_load(src + i);
  }
}

template <bool BF16>
__device__ __forceinline__ double stage_row_store(int n, void* lds, int tid, int nthreads, const RowRegs<BF16>& rr) {
  double acc = 0.0;
  const int nv = BF16 ? n >> 3 : n >> 2;
#pragma unroll
  for (int k = 0; k < RowRegs<BF16>::N; ++k) {
    const int i = tid + k * nthreads;
    if (i >= nv) continue;
    const u32x4 v = rr.v[k];
    if (!BF16) {
      float* dst = reinterpret_cast<float*>(lds) + (i >> 3) * LDS_F32_STRIDE + (i & 7) * 4;
      *reinterpret_cast<u32x4*>(dst) = v;
      // the elements are copied out before the bit cast: this compiler's
      // __builtin_bit_cast of a vector element (v.y) reads element 0
      const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = (double)__builtin_bit_cast(float, p[e]);
        acc = __builtin_fma(a, a, acc);
      }
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(lds) + (i >> 2) * LDS_BF16_STRIDE + (i & 3) * 8;
      *reinterpret_cast<u32x4*>(dst) = v;
      const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = (double)__builtin_bit_cast(float, p[e] << 16);
        const double b = (double)__builtin_bit_cast(float, p[e] & 0xffff0000u);
        acc = __builtin_fma(a, a, acc);
        acc = __builtin_fma(b, b, acc);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, WAVE);
  return acc;
}

// Reads group g of the staged row. The empty asm is a compiler barrier: a
// group is re-read from LDS when needed again instead of being kept live in
// VGPRs.
template <bool BF16>
__device__ __forceinline__ void load_group(const void* lds, int g, float (&x)[QK]) {
  asm volatile("" ::: "memory");
  if (!BF16) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(lds) + g * LDS_F32_STRIDE);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f32x4 v = p[k];
      x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(lds) + g * LDS_BF16_STRIDE);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4 v = p[k];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * k + 2 * h] = __builtin_bit_cast(float, w4[h] << 16);
        x[8 * k + 2 * h + 1] = __builtin_bit_cast(float, w4[h] & 0xffff0000u);
      }
    }
  }
}

// Importances of one 32-weight group [WT 一]: w = q * sqrt(fma(x, x, sigma2)),
// q taken from the element's own column (q == nullptr: q = 1). The range
// test is uniform over the row, so each group takes one branch.
template <bool NORMAL>
__device__ __forceinline__ void group_importances_(const float (&x)[QK], const float* __restrict__ q,
                                                   float sigma2, float (&w)[QK]) {
  if (q) {
    const f32x4* q4 = reinterpret_cast<const f32x4*>(q);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = q4[k];
      w[4 * k] = v.x * sqrt_cr(fma_(x[4 * k], x[4 * k], sigma2), NORMAL);
      w[4 * k + 1] = v.y * sqrt_cr(fma_(x[4 * k + 1], x[4 * k + 1], sigma2), NORMAL);
      w[4 * k + 2] = v.z * sqrt_cr(fma_(x[4 * k + 2], x[4 * k + 2], sigma2), NORMAL);
      w[4 * k + 3] = v.w * sqrt_cr(fma_(x[4 * k + 3], x[4 * k + 3], sigma2), NORMAL);
    }
  } else {
#pragma unroll
    for (int i = 0; i < QK; ++i) w[i] = sqrt_cr(fma_(x[i], x[i], sigma2), NORMAL);
  }
}

// What a row's importances depend on besides x and q.
struct RowImp {
  float sigma2;  // row statistic
  float sigma;   // its correctly rounded square root (the sigma + |x| form)
  bool normal;   // sigma2 in the range of the fast correctly rounded root
  int mode;      // weighting (qr_weighting); always 0 in the default kernels
};

// The other weightings [WT 一, 二]: w = q * m(x) with m one of the magnitude
// forms the pages list as tried before sqrt(sigma2 + x^2), or m = 1 (the
// imatrix alone).
template <int MODE>
__device__ __forceinline__ float magnitude(float x, const RowImp& r) {
  if (MODE == QR_W_X2) return x * x;
  if (MODE == QR_W_ABS_X) return fabsf(x);
  if (MODE == QR_W_SIGMA2_PLUS_X2) return fma_(x, x, r.sigma2);
  if (MODE == QR_W_SIGMA_PLUS_ABS_X) return r.sigma + fabsf(x);
  return 1.0f;
}

template <int MODE>
__device__ __forceinline__ void group_importances_mode(const float (&x)[QK], const float* __restrict__ q,
                                                       const RowImp& r, float (&w)[QK]) {
  if (q) {
    const f32x4* q4 = reinterpret_cast<const f32x4*>(q);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = q4[k];
      w[4 * k] = v.x * magnitude<MODE>(x[4 * k], r);
      w[4 * k + 1] = v.y * magnitude<MODE>(x[4 * k + 1], r);
      w[4 * k + 2] = v.z * magnitude<MODE>(x[4 * k + 2], r);
      w[4 * k + 3] = v.w * magnitude<MODE>(x[4 * k + 3], r);
    }
  } else {
#pragma unroll
    for (int i = 0; i < QK; ++i) w[i] = magnitude<MODE>(x[i], r);
  }
}

// VAR: the kernel takes a weighting at run time (uniform over the launch);
// otherwise it is compiled for the pages' form only.
template <bool VAR>
__device__ __forceinline__ void group_importances(const float (&x)[QK], const float* __restrict__ q,
                                                  const RowImp& r, float (&w)[QK]) {
  if (VAR && r.mode != QR_W_SQRT_SIGMA2_X2) {
    switch (r.mode) {
      case QR_W_X2: group_importances_mode<QR_W_X2>(x, q, r, w); break;
      case QR_W_ABS_X: group_importances_mode<QR_W_ABS_X>(x, q, r, w); break;
      case QR_W_SIGMA2_PLUS_X2: group_importances_mode<QR_W_SIGMA2_PLUS_X2>(x, q, r, w); break;
      case QR_W_SIGMA_PLUS_ABS_X: group_importances_mode<QR_W_SIGMA_PLUS_ABS_X>(x, q, r, w); break;
      default: group_importances_mode<QR_W_IMATRIX_ONLY>(x, q, r, w); break;
    }
    return;
  }
  if (r.normal) group_importances_<true>(x, q, r.sigma2, w);
  else group_importances_<false>(x, q, r.sigma2, w);
}

// Importances with q = 1 for elements OFF .. OFF+N-1 only, written in place
// (the fallback of a sub-block that has no importance at all): the values
// group_importances gives those elements without an imatrix.
template <bool VAR, int OFF, int N>
__device__ __forceinline__ void unit_importances(const float (&x)[QK], const RowImp& r, float (&w)[QK]) {
  auto fill = [&](auto m) {
#pragma unroll
    for (int i = OFF; i < OFF + N; ++i) w[i] = m(x[i]);
  };
  if (VAR && r.mode != QR_W_SQRT_SIGMA2_X2) {
    switch (r.mode) {
      case QR_W_X2: fill([&](float v) { return magnitude<QR_W_X2>(v, r); }); break;
      case QR_W_ABS_X: fill([&](float v) { return magnitude<QR_W_ABS_X>(v, r); }); break;
      case QR_W_SIGMA2_PLUS_X2: fill([&](float v) { return magnitude<QR_W_SIGMA2_PLUS_X2>(v, r); }); break;
      case QR_W_SIGMA_PLUS_ABS_X: fill([&](float v) { return magnitude<QR_W_SIGMA_PLUS_ABS_X>(v, r); }); break;
      default: fill([&](float v) { return magnitude<QR_W_IMATRIX_ONLY>(v, r); }); break;
    }
    return;
  }
  if (r.normal) fill([&](float v) { return sqrt_cr(fma_(v, v, r.sigma2), true); });
  else fill([&](float v) { return sqrt_cr(fma_(v, v, r.sigma2), false); });
}

// -------------------------------------------------------------------------
// greedy flip pass [WT 一]
//
// Fit y ~ d*l with d = A/B, A = sum w y l, B = sum w l^2. Element j moves one
// level along s = sign(A) * sign(y_j*B - l_j*A) (the sign of the pages'
// gradient); the move is kept iff A'^2 * B > A^2 * B' and B' > 0, with
// A' = A + s*w_j*y_j and B' = B + w_j*(2*s*l_j + 1). A pass that keeps no
// move ends the loop for the wave; lanes that kept none repeat a pass whose
// every decision is unchanged, so their result is the same.
//
// The pass covers elements OFF .. OFF+N-1. yw(j, y, wy) gives y_j and the
// product w_j*y_j: the solvers form them from arrays they hold anyway, so no
// 32-wide array of either stays live (that is what keeps the solvers within
// 128 VGPRs, four waves per SIMD).
template <int F, bool ZERO_LO, int OFF = 0, int N = QK, class YW>
__device__ __forceinline__ void flip_passes(YW yw, const float (&w)[QK], float lo, float hi, float (&L)[QK],
                                            float& A_io, float& B_io) {
  float A = A_io, B = B_io;
  auto pass = [&]() {
    bool changed = false;
#pragma unroll
    for (int j = OFF; j < OFF + N; ++j) {
      float y, wy;
      yw(j, y, wy);
      const float t = L[j] * A;
      const float e = fma_(y, B, -t);
      const float sg = __builtin_bit_cast(float, fbits(A) ^ fbits(e));   // sign: sign(A) * sign(e)
      const float s = __builtin_copysignf(1.0f, sg);    // +-1
      const float s2 = s + s;                           // +-2, exactly
      const float lp = L[j] + s;
      const float A1 = fma_(s, wy, A);
      const float B1 = fma_(w[j], fma_(s2, L[j], 1.0f), B);
      // levels [0, hi]: lp >= +0 and lp <= hi is one unsigned compare of
      // the bit patterns (lp is never -0 here; negative values compare high)
      const bool in_range = ZERO_LO ? (fbits(lp) <= fbits(hi)) : ((lp >= lo) && (lp <= hi));
      const bool keep = ((A1 * A1) * B > (A * A) * B1) && (B1 > 0.0f) && in_range;
      A = keep ? A1 : A;
      B = keep ? B1 : B;
      L[j] = keep ? lp : L[j];
      changed |= keep;
    }
    return changed;
  };
  if constexpr (F == 1) {
    // one pass, straight-line: no loop out of which y_j and w_j*y_j could be
    // hoisted into 32-wide arrays
    pass();
  } else {
#pragma unroll 1
    for (int p = 0; p < F; ++p)
      if (!__any(pass())) break;
  }
  A_io = A;
  B_io = B;
}

// -------------------------------------------------------------------------
// symmetric group: levels -NMAX .. NMAX-1, one scale

// Symmetric fit of elements OFF .. OFF+N-1 of a group: the whole group for
// the 32-weight types, a 16-weight sub-block of Q6_K.
//
// The products w*x live only while the trials run; the flip pass forms them
// again rather than keeping that array live next to the levels.
template <int NMAX, int OFF, int N>
__device__ __forceinline__ float sym_fit_part(const float (&x)[QK], const float (&w)[QK], float (&L)[QK]) {
  constexpr float LO = (float)-NMAX, HI = (float)(NMAX - 1);
  // element of largest magnitude, first one on ties: from max and min, with
  // a scan only when +a and -a are both present
  float xmax = x[OFF], xmin = x[OFF];
#pragma unroll
  for (int i = OFF + 1; i < OFF + N; ++i) { xmax = fmaxf(xmax, x[i]); xmin = fminf(xmin, x[i]); }
  const float amax = fmaxf(xmax, -xmin);
  float xm = (xmax > -xmin) ? xmax : xmin;
  if (xmax == -xmin) {
    xm = x[OFF + N - 1];
#pragma unroll
    for (int i = OFF + N - 2; i >= OFF; --i) xm = (fabsf(x[i]) == amax) ? x[i] : xm;
  }
  // Trial scales: the largest element maps to -(NMAX + step*k); each trial
  // is scored by sumlx^2/suml2, compared by cross multiplication in double.
  bool have = false;
  float bS1 = 0.0f, bS2 = 0.0f, bis = 0.0f;
  if (amax > 0.0f) {
    float wx[QK];
#pragma unroll
    for (int i = OFF; i < OFF + N; ++i) wx[i] = w[i] * x[i];
#pragma unroll
    for (int k = 0; k < SYM_CAND; ++k) {
      const float is = -((float)NMAX + CAND_STEP * (float)cand_offset(k)) / xm;
      float S1 = 0.0f, S2 = 0.0f;
#pragma unroll
      for (int i = OFF; i < OFF + N; ++i) {
        const float l = med3(rne(x[i] * is), LO, HI);
        S1 = fma_(wx[i], l, S1);
        S2 = fma_(w[i] * l, l, S2);
      }
      const bool ok = __builtin_isfinite(is) && (S2 > 0.0f);
      const bool better = ok && (!have || ((double)S1 * (double)S1) * (double)bS2 >
                                              ((double)bS1 * (double)bS1) * (double)S2);
      if (better) { have = true; bS1 = S1; bS2 = S2; bis = is; }
    }
  }
  // Without a usable trial, bis = 0 gives zero levels (x is finite) and
  // A = B = 0 lets the flip pass keep no move; the scale is then 0.
#pragma unroll
  for (int i = OFF; i < OFF + N; ++i) L[i] = med3(rne(x[i] * bis), LO, HI);
  float A = bS1, B = bS2;
  flip_passes<SYM_FLIP_PASSES, false, OFF, N>(
      [&](int j, float& y, float& wy) { y = x[j]; wy = w[j] * fresh(x[j]); }, w, LO, HI, L, A, B);
  return have ? A / B : 0.0f;
}

// A whole 32-weight group: importances (with the fallback to q = 1 for a
// group that has none), then the fit.
template <int NMAX, bool BF16, bool VAR>
__device__ __forceinline__ float solve_sym(const void* lds, int g, const float* __restrict__ q, const RowImp& imp,
                                           float (&L)[QK]) {
  float x[QK], w[QK];
  load_group<BF16>(lds, g, x);
  group_importances<VAR>(x, q, imp, w);
  {  // a group with no importance at all falls back to q = 1
    uint32_t any = 0;
#pragma unroll
    for (int i = 0; i < QK; ++i) any |= fbits(w[i]) & 0x7fffffffu;
    if (any == 0) group_importances<VAR>(x, nullptr, imp, w);
  }
  return sym_fit_part<NMAX, 0, QK>(x, w, L);
}

// -------------------------------------------------------------------------
// asymmetric group: levels 0 .. NMAX, x ~ d*l + m

// Two-parameter weighted least squares in double from the five float sums;
// returns the score sum w x^2 - error. Codes with weighted spread below
// 2^-16 of sum w l^2 count as constant; K4 forbids a positive offset.
template <bool K4>
__device__ __forceinline__ void fit_dm(float Sw_, float Sx_, float Sl_, float Sll_, float Slx_,
                                       double& d, double& m, double& score) {
  const double Sw = Sw_, Sx = Sx_, Sl = Sl_, Sll = Sll_, Slx = Slx_;
  const double D = Sw * Sll - Sl * Sl;
  double dd, mm;
  if (D > Sw * Sll * 0x1p-16) {
    const double r = 1.0 / D;
    dd = (Sw * Slx - Sl * Sx) * r;
    mm = (Sll * Sx - Sl * Slx) * r;
  } else {
    dd = 0.0;
    mm = Sx / Sw;
  }
  if (K4 && mm > 0.0) {
    mm = 0.0;
    dd = Sll > 0.0 ? Slx / Sll : 0.0;
  }
  d = dd;
  m = mm;
  score = dd * Slx + mm * Sx;
}

// Returns (d, m) and the levels. The trials run in one sweep over the
// elements with one set of sums per trial (each sum still in ascending
// element order); only x, w and the levels are held as 32-wide arrays, w*x,
// x - lo and x - m being formed again where needed, with the same roundings.
template <int NMAX, bool K4, bool BF16, bool VAR>
__device__ __forceinline__ void solve_asym(const void* lds, int g, const float* __restrict__ q, const RowImp& imp,
                                           float (&L)[QK], float& d_out, float& m_out, float& sw_out) {
  constexpr float HI = (float)NMAX;
  float x[QK], w[QK];
  load_group<BF16>(lds, g, x);
  group_importances<VAR>(x, q, imp, w);
  float Sw = 0.0f;
#pragma unroll
  for (int i = 0; i < QK; ++i) Sw = Sw + w[i];
  if (!(Sw > 0.0f)) {   // no importance at all: q = 1 for this group
    group_importances<VAR>(x, nullptr, imp, w);
    Sw = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) Sw = Sw + w[i];
  }
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < QK; ++i) { lo = fminf(lo, x[i]); hi = fmaxf(hi, x[i]); }
  lo = lo + 0.0f;   // a zero bound is +0 whichever zero min/max returned
  hi = hi + 0.0f;
  if (K4) lo = fminf(lo, 0.0f);
  sw_out = Sw;      // the group's total importance (after any fallback)

  // A constant group (range 0: no finite trial) or importances that
  // underflow to 0 have no usable trial; they take the path below with zero
  // levels and return d = 0, m = lo.
  const float range = hi - lo;
  float is[ASYM_CAND], Sl[ASYM_CAND], Sll[ASYM_CAND], Slx[ASYM_CAND];
#pragma unroll
  for (int k = 0; k < ASYM_CAND; ++k) {
    is[k] = ((float)NMAX + CAND_STEP * (float)cand_offset(k)) / range;
    Sl[k] = 0.0f;
    Sll[k] = 0.0f;
    Slx[k] = 0.0f;
  }
  float Sx = 0.0f;
#pragma unroll
  for (int i = 0; i < QK; ++i) {
    const float wx = w[i] * x[i];
    const float xs = x[i] - lo;
    Sx = Sx + wx;
    // 0 <= xs <= range, so rint(xs * is) lies in [0, NMAX] for these
    // trials and the clamp to the level range never acts.
#pragma unroll
    for (int k = 0; k < ASYM_CAND; ++k) {
      const float l = rne(xs * is[k]);
      const float wl = w[i] * l;
      Sl[k] = Sl[k] + wl;
      Sll[k] = fma_(wl, l, Sll[k]);
      Slx[k] = fma_(wx, l, Slx[k]);
    }
    __builtin_amdgcn_sched_barrier(0);   // element by element: no 32-wide temporaries
  }
  // all sums complete here, before the branches of the fits below
  Sx = fresh(Sx);
#pragma unroll
  for (int k = 0; k < ASYM_CAND; ++k) {
    Sl[k] = fresh(Sl[k]);
    Sll[k] = fresh(Sll[k]);
    Slx[k] = fresh(Slx[k]);
  }
  bool have = false;
  float bis = 0.0f, bSl = 0.0f, bSll = 0.0f, bSlx = 0.0f;
  double bm = 0.0, bscore = 0.0;
#pragma unroll
  for (int k = 0; k < ASYM_CAND; ++k) {
    double d, m, score;
    fit_dm<K4>(Sw, Sx, Sl[k], Sll[k], Slx[k], d, m, score);
    const bool ok = __builtin_isfinite(is[k]) && (Sw > 0.0f);
    if (ok && (!have || score > bscore)) {
      have = true; bis = is[k]; bm = m; bscore = score; bSl = Sl[k]; bSll = Sll[k]; bSlx = Slx[k];
    }
  }
  // Without a usable trial, bis = 0 gives zero levels (0 <= x - lo, finite)
  // and A = B = 0 lets the flip pass keep no move.
  const float lo_ = fresh(lo);
#pragma unroll
  for (int i = 0; i < QK; ++i) L[i] = rne((x[i] - lo_) * bis);

  // flips with the offset of the winning trial held fixed, then a joint refit
  const float mf = (float)bm;
  float A = fma_(-mf, bSl, bSlx), B = bSll;
  flip_passes<ASYM_FLIP_PASSES, true>(
      [&](int j, float& y, float& wy) { y = x[j] - mf; wy = w[j] * y; }, w, 0.0f, HI, L, A, B);

  float Slf = 0.0f;
#pragma unroll
  for (int i = 0; i < QK; ++i) Slf = Slf + w[i] * L[i];
  double d, m, score;
  fit_dm<K4>(Sw, Sx, Slf, B, fma_(mf, Slf, A), d, m, score);
  d_out = have ? (float)d : 0.0f;
  m_out = have ? (float)m : lo;
}

// -------------------------------------------------------------------------
// weighted fit of the eight Q4_K/Q5_K sub-scales (or sub-offsets) [WT 一 applied
// to the values of a super-block]: v_j ~ d * l_j, l_j in 0..63, weights W_j.
// Trial scales map the largest value to 63 + step*k; levels are rounded in
// float; the sums, the score comparisons and the flips run in double (one
// sub-block can carry most of the weight, and the fit's error is then a
// small difference of large scores); d = sumlx/suml2 rounded to float.

__device__ __forceinline__ void fit_levels_pos8(const float (&v)[8], const float (&W)[8], float (&L)[8],
                                                float& d_out) {
  float vmax = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) vmax = fmaxf(vmax, v[i]);
  double Wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) Wv[i] = (double)W[i] * (double)v[i];   // exact
  bool have = false;
  double bS1 = 0.0, bS2 = 0.0;
  float bis = 0.0f;
  if (vmax > 0.0f) {
#pragma unroll
    for (int k = 0; k < SYM_CAND; ++k) {
      const float c = 63.0f + CAND_STEP * (float)cand_offset(k);
      const float is = c / vmax;
      double S1 = 0.0, S2 = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double l = (double)med3(rne(v[i] * is), 0.0f, 63.0f);
        S1 = __builtin_fma(Wv[i], l, S1);
        S2 = __builtin_fma((double)W[i] * l, l, S2);
      }
      const bool ok = __builtin_isfinite(is) && (S2 > 0.0);
      if (ok && (!have || (S1 * S1) * bS2 > (bS1 * bS1) * S2)) {
        have = true; bS1 = S1; bS2 = S2; bis = is;
      }
    }
  }
  if (!have) {
#pragma unroll
    for (int i = 0; i < 8; ++i) L[i] = 0.0f;
    d_out = 0.0f;
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) L[i] = med3(rne(v[i] * bis), 0.0f, 63.0f);
  double A = bS1, B = bS2;
#pragma unroll 1
  for (int p = 0; p < SYM_FLIP_PASSES; ++p) {
    bool changed = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double e = __builtin_fma((double)v[j], B, -((double)L[j] * A));
      const double sg = (__builtin_signbit(A) != __builtin_signbit(e)) ? -1.0 : 1.0;
      const double lp = (double)L[j] + sg;
      const double A1 = __builtin_fma(sg, Wv[j], A);
      const double B1 = __builtin_fma((double)W[j], __builtin_fma(2.0 * sg, (double)L[j], 1.0), B);
      const bool keep = ((A1 * A1) * B > (A * A) * B1) && (B1 > 0.0) && (lp >= 0.0) && (lp <= 63.0);
      A = keep ? A1 : A;
      B = keep ? B1 : B;
      L[j] = keep ? (float)lp : L[j];
      changed |= keep;
    }
    if (!changed) break;
  }
  d_out = (float)(A / B);
}

// -------------------------------------------------------------------------
// packers

// 32 codes in [0, 15] -> 16 bytes: byte i = u_i | u_{i+16} << 4.
__device__ __forceinline__ uint4 pack_nibbles(const uint32_t (&u)[QK]) {
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = 4 * k + b;
      v |= ((u[i] & 15u) | ((u[i + 16] & 15u) << 4)) << (8 * b);
    }
    o[k] = v;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Same layout from codes held as floats (exact small integers): each byte
// u_i + 16*u_{i+16} is formed in float and converted into place.
__device__ __forceinline__ uint4 pack_nibbles_f(const float (&u)[QK]) {
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = 4 * k + b;
      v = __builtin_amdgcn_cvt_pk_u8_f32(fma_(16.0f, u[i + 16], u[i]), b, v);
    }
    o[k] = v;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint32_t pack_high_bits(const uint32_t (&u)[QK]) {
  uint32_t qh = 0;
#pragma unroll
  for (int i = 0; i < QK; ++i) qh |= ((u[i] >> 4) & 1u) << i;
  return qh;
}

__device__ __forceinline__ void store_u32(uint8_t* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }

// -------------------------------------------------------------------------
// weight-row kernel: one workgroup of W waves per row (W = ceil(groups/64),
// at most MAX_ROW_WAVES); every lane solves groups tid, tid + 64W, ...

constexpr int MAX_ROW_WAVES = 8;
constexpr int LDS_PER_WORKGROUP = 160 * 1024;
static_assert((size_t)QR_MAX_ROW_F32 / QK * LDS_F32_STRIDE * 4 + 8 * MAX_ROW_WAVES <= LDS_PER_WORKGROUP &&
                  (size_t)QR_MAX_ROW_BF16 / QK * LDS_BF16_STRIDE * 2 + 8 * MAX_ROW_WAVES <= LDS_PER_WORKGROUP,
              "the longest row and the partial sums fit in one workgroup's LDS");

// Waves per SIMD the register allocation aims at: four (the LDS limit of a
// 4096-value fp32 row). The solvers keep three 32-wide arrays live (x, w and
// the levels), which fits in 128 VGPRs without spills.
__host__ __device__ constexpr int row_waves_per_eu(int) { return 4; }

// Solves group g of a staged row (lds: the row's staged groups) with the
// imatrix entries qg of its columns (nullptr: q = 1) and writes its packed
// bytes into orow. For the K types lanes 8s .. 8s+7 must hold the eight
// groups of one super-block, all active: they combine their scales.
template <int TYPE, bool BF16, bool VAR>
__device__ __forceinline__ void quantize_group(const void* lds, int g, const float* __restrict__ qg,
                                               const RowImp& imp, uint8_t* __restrict__ orow, int fit) {
  float L[QK];

  if constexpr (TYPE == QR_Q6_K) {  // lanes 8s .. 8s+7: the eight 32-weight groups of a super-block
    float x[QK], w[QK];
    load_group<BF16>(lds, g, x);
    group_importances<VAR>(x, qg, imp, w);
    {  // a sub-block (16 weights) with no importance at all falls back to q = 1
      uint32_t any0 = 0, any1 = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        any0 |= fbits(w[i]) & 0x7fffffffu;
        any1 |= fbits(w[16 + i]) & 0x7fffffffu;
      }
      if (any0 == 0) unit_importances<VAR, 0, 16>(x, imp, w);
      if (any1 == 0) unit_importances<VAR, 16, 16>(x, imp, w);
    }
    const float d0 = sym_fit_part<32, 0, 16>(x, w, L);    // sub-block 2j
    const float d1 = sym_fit_part<32, 16, 16>(x, w, L);   // sub-block 2j+1
    const float amx = oct_max(fmaxf(fabsf(d0), fabsf(d1)));   // over the super-block's 16 sub-blocks
    const _Float16 d16 = (_Float16)(amx / 127.0f);
    const float dA = (float)d16;
    const float s0 = dA > 0.0f ? med3(rne(d0 / dA), -127.0f, 127.0f) : 0.0f;
    const float s1 = dA > 0.0f ? med3(rne(d1 / dA), -127.0f, 127.0f) : 0.0f;
    const float ds0 = dA * s0, ds1 = dA * s1;   // exact: 11-bit times 8-bit
    const float id0 = ds0 == 0.0f ? 0.0f : 1.0f / ds0;
    const float id1 = ds1 == 0.0f ? 0.0f : 1.0f / ds1;
    uint32_t u[QK];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u[i] = ds0 == 0.0f ? 32u : (uint32_t)(int32_t)(med3(rne(x[i] * id0), -32.0f, 31.0f) + 32.0f);
      u[16 + i] = ds1 == 0.0f ? 32u : (uint32_t)(int32_t)(med3(rne(x[16 + i] * id1), -32.0f, 31.0f) + 32.0f);
    }
    uint32_t h0 = 0, h1 = 0;  // bits 4 and 5 of each code, two bits apiece
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h0 |= ((u[i] >> 4) & 3u) << (2 * i);
      h1 |= ((u[16 + i] >> 4) & 3u) << (2 * i);
    }
    const uint4 qs = pack_nibbles(u);
    const int j = g & 7;
    uint8_t* p = orow + (size_t)(g >> 3) * 212;
    // sub-scales: lane j holds bytes 2j, 2j+1; even lanes write a word
    const uint32_t v16 = ((uint32_t)(int32_t)s0 & 255u) | (((uint32_t)(int32_t)s1 & 255u) << 8);
    const uint32_t pair = (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)v16);
    if ((j & 1) == 0) store_u32(p + 4 + 2 * j, v16 | (pair << 16));
    if (j == 0) store_u32(p, (uint32_t)__builtin_bit_cast(uint16_t, d16));   // d16, then the zero pad
    uint8_t* pq = p + 20 + 16 * j;
    store_u32(pq, qs.x); store_u32(pq + 4, qs.y); store_u32(pq + 8, qs.z); store_u32(pq + 12, qs.w);
    store_u32(p + 148 + 8 * j, h0);
    store_u32(p + 152 + 8 * j, h1);
  } else if constexpr (TYPE == QR_Q6_0) {
    const float d = solve_sym<32, BF16, VAR>(lds, g, qg, imp, L);
    uint32_t u[QK];
#pragma unroll
    for (int i = 0; i < QK; ++i) u[i] = (uint32_t)(int32_t)(L[i] + 32.0f);
    uint32_t h0 = 0, h1 = 0;  // bits 4 and 5 of each code, two bits apiece
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h0 |= ((u[i] >> 4) & 3u) << (2 * i);
      h1 |= ((u[16 + i] >> 4) & 3u) << (2 * i);
    }
    const uint4 qs = pack_nibbles(u);
    uint8_t* p = orow + (size_t)g * 28;
    store_u32(p, fbits(d));
    store_u32(p + 4, h0); store_u32(p + 8, h1);
    store_u32(p + 12, qs.x); store_u32(p + 16, qs.y); store_u32(p + 20, qs.z); store_u32(p + 24, qs.w);
  } else if constexpr (TYPE == QR_Q4_0 || TYPE == QR_Q5_0) {
    constexpr int NMAX = TYPE == QR_Q4_0 ? 8 : 16;
    const float d = solve_sym<NMAX, BF16, VAR>(lds, g, qg, imp, L);
    if constexpr (TYPE == QR_Q4_0) {
      float uf[QK];
#pragma unroll
      for (int i = 0; i < QK; ++i) uf[i] = L[i] + (float)NMAX;
      const uint4 qs = pack_nibbles_f(uf);
      uint8_t* p = orow + (size_t)g * 20;
      store_u32(p, fbits(d));
      store_u32(p + 4, qs.x); store_u32(p + 8, qs.y); store_u32(p + 12, qs.z); store_u32(p + 16, qs.w);
    } else {
      uint32_t u[QK];
#pragma unroll
      for (int i = 0; i < QK; ++i) u[i] = (uint32_t)(int32_t)(L[i] + (float)NMAX);
      const uint4 qs = pack_nibbles(u);
      uint8_t* p = orow + (size_t)g * 24;
      store_u32(p, fbits(d));
      store_u32(p + 4, pack_high_bits(u));
      store_u32(p + 8, qs.x); store_u32(p + 12, qs.y); store_u32(p + 16, qs.z); store_u32(p + 20, qs.w);
    }
  } else if constexpr (TYPE == QR_Q4_1 || TYPE == QR_Q5_1) {
    constexpr int NMAX = TYPE == QR_Q4_1 ? 15 : 31;
    float d, m;
    float sw;
    solve_asym<NMAX, false, BF16, VAR>(lds, g, qg, imp, L, d, m, sw);
    if constexpr (TYPE == QR_Q4_1) {
      const uint4 qs = pack_nibbles_f(L);
      uint8_t* p = orow + (size_t)g * 24;
      store_u32(p, fbits(d)); store_u32(p + 4, fbits(m));
      store_u32(p + 8, qs.x); store_u32(p + 12, qs.y); store_u32(p + 16, qs.z); store_u32(p + 20, qs.w);
    } else {
      uint32_t u[QK];
#pragma unroll
      for (int i = 0; i < QK; ++i) u[i] = (uint32_t)L[i];
      const uint4 qs = pack_nibbles(u);
      uint8_t* p = orow + (size_t)g * 28;
      store_u32(p, fbits(d)); store_u32(p + 4, fbits(m));
      store_u32(p + 8, pack_high_bits(u));
      store_u32(p + 12, qs.x); store_u32(p + 16, qs.y); store_u32(p + 20, qs.z); store_u32(p + 24, qs.w);
    }
  } else {  // QR_Q4_K, QR_Q5_K: lanes 8s .. 8s+7 hold the sub-blocks of one super-block [KQ 一]
    constexpr int KMAX = TYPE == QR_Q5_K ? 31 : 15;    // levels 0..KMAX
    constexpr int KBYTES = TYPE == QR_Q5_K ? 176 : 144;
    float d, m, sw;
    solve_asym<KMAX, true, BF16, VAR>(lds, g, qg, imp, L, d, m, sw);
    const float a = d > 0.0f ? d : 0.0f;
    const float b = -m > 0.0f ? -m : 0.0f;
    const int j = g & 7;
    _Float16 d16, m16;
    float sc, mn;
    if (VAR && fit == QR_FIT_WEIGHTED) {
      // lanes 0-3 of the super-block fit the eight scales, lanes 4-7 the
      // eight offsets (the same instructions on other data); lanes 0 and
      // 4 then hand out their levels, four to a word, and their scales
      const bool offs = (j & 4) != 0;
      float vv[8], wv[8], lv[8], dv;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float ak = __shfl(a, k, 8), bk = __shfl(b, k, 8);
        vv[k] = offs ? bk : ak;
        wv[k] = __shfl(sw, k, 8);
      }
      fit_levels_pos8(vv, wv, lv, dv);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w0 |= (uint32_t)lv[k] << (8 * k);
        w1 |= (uint32_t)lv[4 + k] << (8 * k);
      }
      const uint32_t sw0 = __shfl(w0, 0, 8), sw1 = __shfl(w1, 0, 8);
      const uint32_t mw0 = __shfl(w0, 4, 8), mw1 = __shfl(w1, 4, 8);
      const float da = __shfl(dv, 0, 8), db = __shfl(dv, 4, 8);
      d16 = (_Float16)da;
      m16 = (_Float16)db;
      sc = (float)(((j < 4 ? sw0 : sw1) >> (8 * (j & 3))) & 255u);
      mn = (float)(((j < 4 ? mw0 : mw1) >> (8 * (j & 3))) & 255u);
      if ((float)d16 == 0.0f) sc = 0.0f;
      if ((float)m16 == 0.0f) mn = 0.0f;
    } else {
      const float A = oct_max(a), Bm = oct_max(b);   // the super-block's largest scale and offset
      d16 = (_Float16)(A / 63.0f);
      m16 = (_Float16)(Bm / 63.0f);
      const float dA0 = (float)d16, dB0 = (float)m16;
      sc = dA0 > 0.0f ? med3(rne(a / dA0), 0.0f, 63.0f) : 0.0f;
      mn = dB0 > 0.0f ? med3(rne(b / dB0), 0.0f, 63.0f) : 0.0f;
    }
    const float dA = (float)d16, dB = (float)m16;
    const float ds = dA * sc, dm = dB * mn;
    float u[QK];
    if (ds == 0.0f) {
#pragma unroll
      for (int i = 0; i < QK; ++i) u[i] = 0.0f;
    } else {
      const float id = 1.0f / ds;
      load_group<BF16>(lds, g, u);
#pragma unroll
      for (int i = 0; i < QK; ++i) u[i] = med3(rne((u[i] + dm) * id), 0.0f, (float)KMAX);
    }
    uint8_t* p = orow + (size_t)(g >> 3) * KBYTES;
    if constexpr (TYPE == QR_Q5_K) {   // fifth bits at 16 + 4j, low nibbles at 48 + 16j
      uint32_t ui[QK];
#pragma unroll
      for (int i = 0; i < QK; ++i) ui[i] = (uint32_t)u[i];
      store_u32(p + 16 + 4 * j, pack_high_bits(ui));
      *reinterpret_cast<uint4*>(p + 48 + 16 * j) = pack_nibbles(ui);
    } else {
      *reinterpret_cast<uint4*>(p + 16 + 16 * j) = pack_nibbles_f(u);
    }
    // the eight 6-bit fields, merged over the super-block's lanes
    const uint64_t scj = (uint64_t)(uint32_t)sc << (6 * j);
    const uint64_t mnj = (uint64_t)(uint32_t)mn << (6 * j);
    const uint64_t scb = (uint64_t)oct_or((uint32_t)scj) | ((uint64_t)oct_or((uint32_t)(scj >> 32)) << 32);
    const uint64_t mnb = (uint64_t)oct_or((uint32_t)mnj) | ((uint64_t)oct_or((uint32_t)(mnj >> 32)) << 32);
    if (j == 0) {
      const uint32_t h0 = (uint32_t)__builtin_bit_cast(uint16_t, d16) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, m16) << 16);
      const uint32_t h1 = (uint32_t)scb;
      const uint32_t h2 = (uint32_t)(scb >> 32) | ((uint32_t)mnb << 16);
      const uint32_t h3 = (uint32_t)(mnb >> 16);
      *reinterpret_cast<uint4*>(p) = make_uint4(h0, h1, h2, h3);
    }
  }
}

template <int TYPE, bool BF16, bool VAR>
__global__ __launch_bounds__(WAVE * MAX_ROW_WAVES) __attribute__((amdgpu_waves_per_eu(row_waves_per_eu(TYPE)))) void k_quantize_rows(const void* __restrict__ x,
                                                                        const float* __restrict__ imatrix,
                                                                        int n_per_row, int64_t rows_per_group,
                                                                        uint8_t* __restrict__ out,
                                                                        int64_t row_bytes, int weighting,
                                                                        int fit) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int64_t row = blockIdx.x;
  const int n_groups = n_per_row / QK;
  const size_t elem = BF16 ? 2 : 4;
  double* partial = reinterpret_cast<double*>(lds_raw + (size_t)n_groups * (BF16 ? 2 * LDS_BF16_STRIDE
                                                                                  : 4 * LDS_F32_STRIDE));

  const void* xrow = reinterpret_cast<const unsigned char*>(x) + (size_t)row * n_per_row * elem;
  const double ss_wave = stage_row<BF16>(xrow, n_per_row, lds_raw, tid, nthreads);
  if ((tid & (WAVE - 1)) == 0) partial[tid / WAVE] = ss_wave;
  __syncthreads();
  double ss = 0.0;
  for (int k = 0; k < nthreads / WAVE; ++k) ss += partial[k];
  const float sigma2 = (float)(ss / (double)n_per_row);
  const bool normal_range = sigma2 >= 0x1p-96f && sigma2 <= 3.0e38f;
  RowImp imp;
  imp.sigma2 = sigma2;
  imp.normal = normal_range;
  imp.mode = VAR ? weighting : QR_W_SQRT_SIGMA2_X2;
  imp.sigma = VAR && weighting == QR_W_SIGMA_PLUS_ABS_X ? sqrt_cr(sigma2, normal_range) : 0.0f;

  const float* q = imatrix ? imatrix + (row / rows_per_group) * (int64_t)n_per_row : nullptr;
  uint8_t* orow = out + row * row_bytes;

  for (int base = 0; base < n_groups; base += nthreads) {
    const int g = base + tid;
    if (g >= n_groups) continue;
    quantize_group<TYPE, BF16, VAR>(lds_raw, g, q ? q + g * QK : nullptr, imp, orow, fit);
  }
}

// Streaming weight-row kernel, for widths whose groups would leave lanes of
// the last wave idle (7168 values: 224 groups on four waves, 32 of 256
// lanes idle). The workgroup's L = 64 W lanes walk blocks of `block_rows`
// consecutive rows as one sequence of groups: pass i gives lane t group
// L i + t of the block, so every lane works (block_rows x groups is a
// multiple of L). Two row slots in LDS hold the rows a pass touches (the
// host checks that a pass spans at most two rows and that each pass needs
// at most one row more than the one before); each row is staged, with its
// statistic, when the first pass that needs it begins, into the slot of
// the row two before it, which no later pass touches. Staging and the
// statistic are those of k_quantize_rows with the same W, so the results
// are the same bytes.
template <int TYPE, bool BF16, bool VAR>
__global__ __launch_bounds__(WAVE * MAX_ROW_WAVES) __attribute__((amdgpu_waves_per_eu(row_waves_per_eu(TYPE)))) void k_quantize_rows_stream(
    const void* __restrict__ x, const float* __restrict__ imatrix, int n_per_row, int64_t n_rows,
    int64_t rows_per_group, uint8_t* __restrict__ out, int64_t row_bytes, int weighting, int fit, int block_rows) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int n_groups = n_per_row / QK;
  const size_t elem = BF16 ? 2 : 4;
  const size_t slot_bytes = (size_t)n_groups * (BF16 ? 2 * LDS_BF16_STRIDE : 4 * LDS_F32_STRIDE);
  double* partial = reinterpret_cast<double*>(lds_raw + 2 * slot_bytes);
  const int64_t row0 = (int64_t)blockIdx.x * block_rows;
  const int rows = (int)(n_rows - row0 < block_rows ? n_rows - row0 : block_rows);
  const int passes = (int)(((int64_t)rows * n_groups + nthreads - 1) / nthreads);
  float sig0 = 0.0f, sig1 = 0.0f;   // the statistic of the row in each slot

  // stages block row r into slot r & 1 and keeps its statistic; the row's
  // loads are issued before the barrier, so they overlap the wait for the
  // last waves of the pass before
  auto stage = [&](int r) {
    RowRegs<BF16> rr;
    // the thread's addresses are recomputed here (a few integer
    // instructions) rather than kept live through the passes
    int t = tid;
    asm volatile("" : "+v"(t));
    const void* xrow = reinterpret_cast<const unsigned char*>(x) + (size_t)(row0 + r) * n_per_row * elem;
    stage_row_load<BF16>(xrow, n_per_row, t, nthreads, rr);
    __syncthreads();   // every lane is done with the row the slot held
    const double ss_wave = stage_row_store<BF16>(n_per_row, lds_raw + (r & 1) * slot_bytes, t, nthreads, rr);
    if ((t & (WAVE - 1)) == 0) partial[t / WAVE] = ss_wave;
    __syncthreads();
    double ss = 0.0;
    for (int k = 0; k < nthreads / WAVE; ++k) ss += partial[k];
    // the same value in every lane: kept in a scalar register
    const float s2 = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, (float)(ss / (double)n_per_row))));
    if (r & 1) sig1 = s2;
    else sig0 = s2;
  };
  stage(0);
  int staged = 0;   // the last block row staged
  for (int p = 0; p < passes; ++p) {
    // the last row this pass touches
    int64_t last = ((int64_t)p * nthreads + nthreads - 1) / n_groups;
    if (last > rows - 1) last = rows - 1;
    if (last > staged) {
      stage((int)last);
      staged = (int)last;
    }
    const int64_t gg = (int64_t)p * nthreads + tid;   // group in the block
    const int r = (int)(gg / n_groups);
    if (r >= rows) continue;
    const int g = (int)(gg - (int64_t)r * n_groups);
    const float sigma2 = (r & 1) ? sig1 : sig0;
    const bool normal_range = sigma2 >= 0x1p-96f && sigma2 <= 3.0e38f;
    RowImp imp;
    imp.sigma2 = sigma2;
    imp.normal = normal_range;
    imp.mode = VAR ? weighting : QR_W_SQRT_SIGMA2_X2;
    imp.sigma = VAR && weighting == QR_W_SIGMA_PLUS_ABS_X ? sqrt_cr(sigma2, normal_range) : 0.0f;
    const int64_t row = row0 + r;
    const float* q = imatrix ? imatrix + (row / rows_per_group) * (int64_t)n_per_row : nullptr;
    quantize_group<TYPE, BF16, VAR>(lds_raw + (r & 1) * slot_bytes, g, q ? q + g * QK : nullptr, imp,
                                    out + row * row_bytes, fit);
  }
}

// -------------------------------------------------------------------------
// Q8_K activation kernels [Q8 修复方案; 技术启示与后续演进 for the 64- and
// 16-value blocks]
//
// B/4 lanes own a block of B values (one float4 each): a wave holds 2, 4 or
// 16 consecutive blocks per step and Q8_STEPS steps per iteration (4 KB of
// fp32 input), all loads issued before any use. amax and the code sums are
// reduced over the block's lanes with DPP row operations (one LDS-unit
// shuffle for the last step of a 128-value block). The packed blocks of an
// iteration (a 16-byte aligned run) are assembled in LDS and written with
// coalesced 16-byte stores. With one iteration per wave, the grid gives
// each wave its own chunk (measured on 8192 x 7168 fp32: 2, 4, 8 and 16
// steps reach 0.71, 0.72, 0.69 and 0.66 of HBM peak; 4 or 2 chunks per
// wave are slower still).

constexpr int Q8_STEPS = 4;                      // wave steps per iteration

__host__ __device__ constexpr int q8_block_bytes(int b) { return b == 128 ? 140 : b == 64 ? 72 : 24; }
__host__ __device__ constexpr int q8_chunk_blocks(int b) { return (256 / b) * Q8_STEPS; }

// max over each 32-lane half of the wave
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));   // max over 8
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));        // max over 16
  return fmaxf(v, __shfl_xor(v, 16, 32));        // max over 32
}

// sum over each group of 8 lanes
__device__ __forceinline__ int oct_sum(int v) {
  v += dpp_i<DPP_QUAD_XOR1>(v);
  v += dpp_i<DPP_QUAD_XOR2>(v);
  return v + dpp_i<DPP_ROW_HALF_MIRROR>(v);
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* __restrict__ x, int64_t e) {
  if (!BF16) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + e));
    return make_float4(v.x, v.y, v.z, v.w);
  }
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(x) + e));
  return make_float4(__builtin_bit_cast(float, v.x << 16), __builtin_bit_cast(float, v.x & 0xffff0000u),
                     __builtin_bit_cast(float, v.y << 16), __builtin_bit_cast(float, v.y & 0xffff0000u));
}

// max over each group of 4 lanes
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  return fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
}

// max over each row of 16 lanes
__device__ __forceinline__ float row_max(float v) {
  v = quad_max(v);
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
}

// sum over each group of 4 lanes
__device__ __forceinline__ int quad_sum(int v) {
  v += dpp_i<DPP_QUAD_XOR1>(v);
  return v + dpp_i<DPP_QUAD_XOR2>(v);
}

template <int B>
__device__ __forceinline__ float block_max(float v) {
  if constexpr (B == 128) return half_wave_max(v);
  else if constexpr (B == 64) return row_max(v);
  else return quad_max(v);
}

template <int B, bool BF16>
__global__ __launch_bounds__(256) void k_quantize_q8k(const void* __restrict__ x, int64_t n_blocks,
                                                      uint8_t* __restrict__ out) {
  constexpr int LPB = B / 4;                       // lanes per block
  constexpr int BPS = WAVE / LPB;                  // blocks per wave step
  constexpr int BW = q8_block_bytes(B) / 4;        // words per packed block
  constexpr int CB = q8_chunk_blocks(B);           // blocks per iteration
  __shared__ __align__(16) uint32_t stage[4][CB * BW];
  const int lane = threadIdx.x & 63;
  const int wib = threadIdx.x >> 6;
  const int sub = lane / LPB;             // which block of a step
  const int lb = lane % LPB;              // 4-value slot inside the block
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  uint32_t* st = stage[wib];

  // rows are contiguous and hold whole blocks, so block b of the whole
  // tensor starts at value B*b and its packed bytes at block_bytes*b
  for (int64_t b0 = wave * CB; b0 < n_blocks; b0 += n_waves * CB) {
    float4 v[Q8_STEPS];
#pragma unroll
    for (int u = 0; u < Q8_STEPS; ++u) {
      const int64_t blk = b0 + BPS * u + sub;
      v[u] = blk < n_blocks ? load4<BF16>(x, blk * B + 4 * lb) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < Q8_STEPS; ++u) {
      float amax = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
      amax = block_max<B>(amax);
      const float id = amax > 0.0f ? 127.0f / amax : 0.0f;
      const bool zero = !(amax > 0.0f) || !__builtin_isfinite(id);
      const float d = zero ? 0.0f : amax / 127.0f;
      int32_t q0 = 0, q1 = 0, q2 = 0, q3 = 0;
      if (!zero) {
        q0 = (int32_t)med3(rne(v[u].x * id), -127.0f, 127.0f);
        q1 = (int32_t)med3(rne(v[u].y * id), -127.0f, 127.0f);
        q2 = (int32_t)med3(rne(v[u].z * id), -127.0f, 127.0f);
        q3 = (int32_t)med3(rne(v[u].w * id), -127.0f, 127.0f);
      }
      uint32_t* bs = st + BW * (BPS * u + sub);   // this block in the chunk
      bs[1 + lb] = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                   ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
      if (lb == 0) bs[0] = fbits(d);
      if constexpr (B == 16) {
        const int32_t sum = quad_sum(q0 + q1 + q2 + q3);   // the block's 16 codes
        if (lb == 0) bs[5] = (uint32_t)(sum & 0xffff);     // upper half: the zero pad
      } else {
        const int32_t sum = oct_sum(q0 + q1 + q2 + q3);    // sum of group lb/8
        const int32_t s_next = dpp_i<DPP_ROW_SHL8>(sum);   // lanes 0, 16 of a row: the next group
        if (lb == 0 || (B == 128 && lb == 16))
          bs[(B == 128 ? 33 : 17) + (lb >> 4)] = (uint32_t)(sum & 0xffff) | ((uint32_t)(s_next & 0xffff) << 16);
      }
    }
    // one wave's LDS accesses complete in order; the barrier only keeps the
    // compiler from moving the reads above the writes
    __builtin_amdgcn_wave_barrier();
    // 16-byte stores of the chunk (its start block_bytes*b0 is a multiple of
    // 16); plain stores measured 3% faster than nontemporal ones here
    const int64_t nb = (n_blocks - b0) < CB ? (n_blocks - b0) : CB;
    const int nvec = (int)(nb * BW / 4);
    uint8_t* dst = out + b0 * (4 * BW);
    for (int i = lane; i < nvec; i += WAVE)
      reinterpret_cast<u32x4*>(dst)[i] = *reinterpret_cast<const u32x4*>(st + 4 * i);
    if (lane == 0 && (nb * BW) % 4) {                      // a partial last vector (ragged end)
      for (int k = nvec * 4; k < (int)(nb * BW); ++k) reinterpret_cast<uint32_t*>(dst)[k] = st[k];
    }
    __builtin_amdgcn_wave_barrier();
  }
}
static_assert(q8_chunk_blocks(128) * 140 % 16 == 0 && q8_chunk_blocks(64) * 72 % 16 == 0 &&
                  q8_chunk_blocks(16) * 24 % 16 == 0,
              "every iteration's output starts 16-byte aligned");

// -------------------------------------------------------------------------
// decoders: 8 lanes per 32-weight group, one float4 of output each; a wave
// covers 8 groups per step and DQ_STEPS steps per iteration

constexpr int DQ_STEPS = 2;

// Rows are contiguous and hold whole blocks, so packed block B of the tensor
// starts at byte B * block_bytes and 32-weight unit U's output at 32 * U.
// Every word an item needs is loaded before any is used, so an item costs
// one memory round trip.
template <int TYPE>
__device__ __forceinline__ void decode4(const uint8_t* __restrict__ in, int64_t U, int k, float (&o)[4]) {
  if constexpr (TYPE == QR_Q8_K128 || TYPE == QR_Q8_K64 || TYPE == QR_Q8_K16) {
    // values 32U + 4k .. +3: block (32U + 4k) / B, code word ((32U + 4k) % B) / 4
    const uint8_t* blk;
    int off;
    if constexpr (TYPE == QR_Q8_K128) {
      blk = in + (U >> 2) * 140;
      off = 4 + 32 * (int)(U & 3) + 4 * k;
    } else if constexpr (TYPE == QR_Q8_K64) {
      blk = in + (U >> 1) * 72;
      off = 4 + 32 * (int)(U & 1) + 4 * k;
    } else {
      blk = in + (2 * U + (k >> 2)) * 24;
      off = 4 + 4 * (k & 3);
    }
    const uint32_t dbits = *reinterpret_cast<const uint32_t*>(blk);
    const uint32_t qv = *reinterpret_cast<const uint32_t*>(blk + off);
    const float d = __builtin_bit_cast(float, dbits);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = d * (float)(int8_t)(qv >> (8 * i));
  } else if constexpr (TYPE == QR_Q4_K || TYPE == QR_Q5_K) {
    constexpr bool Q5 = TYPE == QR_Q5_K;
    const uint8_t* p = in + (U >> 3) * (Q5 ? 176 : 144);
    const int j = (int)(U & 7);
    const u32x4 h = *reinterpret_cast<const u32x4*>(p);       // 144*B and 176*B are 16-byte aligned
    const uint32_t bytes = *reinterpret_cast<const uint32_t*>(p + (Q5 ? 48 : 16) + 16 * j + 4 * (k & 3));
    const uint32_t qh = Q5 ? *reinterpret_cast<const uint32_t*>(p + 16 + 4 * j) >> (4 * k) : 0u;
    const uint64_t scb = (uint64_t)h.y | ((uint64_t)(h.z & 0xffffu) << 32);
    const uint64_t mnb = (uint64_t)(h.z >> 16) | ((uint64_t)h.w << 16);
    const float dA = (float)__builtin_bit_cast(_Float16, (uint16_t)(h.x & 0xffffu));
    const float dB = (float)__builtin_bit_cast(_Float16, (uint16_t)(h.x >> 16));
    const float ds = dA * (float)(uint32_t)((scb >> (6 * j)) & 63u);
    const float dm = dB * (float)(uint32_t)((mnb >> (6 * j)) & 63u);
    const int sh = (k >> 2) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = fma_(ds, (float)(((bytes >> (8 * i + sh)) & 15u) | (((qh >> i) & 1u) << 4)), -dm);
  } else if constexpr (TYPE == QR_Q6_K) {
    const uint8_t* p = in + (U >> 3) * 212;
    const int j = (int)(U & 7);
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(p);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(p + 4 + 4 * (j >> 1));
    const uint32_t qh = *reinterpret_cast<const uint32_t*>(p + 148 + 8 * j + 4 * (k >> 2));
    const uint32_t bytes = *reinterpret_cast<const uint32_t*>(p + 20 + 16 * j + 4 * (k & 3));
    const float dA = (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xffffu));
    const float ds = dA * (float)(int32_t)(int8_t)(uint8_t)(sw >> (8 * (2 * (j & 1) + (k >> 2))));
    const int sh = (k >> 2) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = ((bytes >> (8 * i + sh)) & 15u) | (((qh >> (2 * (4 * (k & 3) + i))) & 3u) << 4);
      o[i] = ds * (float)((int32_t)u - 32);
    }
  } else if constexpr (TYPE == QR_Q6_0) {
    const uint8_t* p = in + U * 28;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(p);
    const uint32_t qh = *reinterpret_cast<const uint32_t*>(p + 4 + 4 * (k >> 2));  // plane of elements 16*(k/4)..
    const uint32_t bytes = *reinterpret_cast<const uint32_t*>(p + 12 + 4 * (k & 3));
    const float d = __builtin_bit_cast(float, w0);
    const int sh = (k >> 2) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = ((bytes >> (8 * i + sh)) & 15u) | (((qh >> (2 * (4 * (k & 3) + i))) & 3u) << 4);
      o[i] = d * (float)((int32_t)u - 32);
    }
  } else {
    constexpr int BB = TYPE == QR_Q4_0 ? 20 : (TYPE == QR_Q5_1 ? 28 : 24);
    constexpr bool SYM = TYPE == QR_Q4_0 || TYPE == QR_Q5_0;
    constexpr bool FIVE = TYPE == QR_Q5_0 || TYPE == QR_Q5_1;
    constexpr int QS = (SYM ? 4 : 8) + (FIVE ? 4 : 0);          // offset of the nibbles
    const uint8_t* p = in + U * BB;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(p);
    const uint32_t w1 = SYM ? 0u : *reinterpret_cast<const uint32_t*>(p + 4);
    const uint32_t qh = FIVE ? *reinterpret_cast<const uint32_t*>(p + QS - 4) : 0u;
    const uint32_t bytes = *reinterpret_cast<const uint32_t*>(p + QS + 4 * (k & 3));
    const float d = __builtin_bit_cast(float, w0);
    const int sh = (k >> 2) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = (bytes >> (8 * i + sh)) & 15u;
      if (FIVE) u |= ((qh >> (4 * k + i)) & 1u) << 4;
      if constexpr (SYM) o[i] = d * (float)((int32_t)u - (TYPE == QR_Q4_0 ? 8 : 16));
      else o[i] = fma_(d, (float)u, __builtin_bit_cast(float, w1));
    }
  }
}

// n_items = values / 4 (a Q8_K16 tensor may end halfway through a unit)
template <int TYPE>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ in, int64_t n_items,
                                                    float* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  // a wave's steps are adjacent 64-item runs, so that its stores fill
  // DQ_STEPS consecutive KB (measured 5% faster than steps a grid apart)
  const int64_t lane = tid & 63, wv = tid >> 6;
  for (int64_t t0 = wv * 64 * DQ_STEPS + lane; t0 < n_items; t0 += nthreads * DQ_STEPS) {
    float o[DQ_STEPS][4];
#pragma unroll
    for (int s = 0; s < DQ_STEPS; ++s) {
      const int64_t t = t0 + s * 64;
      if (t < n_items) decode4<TYPE>(in, t >> 3, (int)(t & 7), o[s]);
    }
#pragma unroll
    for (int s = 0; s < DQ_STEPS; ++s) {
      const int64_t t = t0 + s * 64;
      if (t < n_items)
        __builtin_nontemporal_store(f32x4{o[s][0], o[s][1], o[s][2], o[s][3]}, reinterpret_cast<f32x4*>(out + 4 * t));
    }
  }
}

// -------------------------------------------------------------------------
// host side


int block_elems(int t) {
  switch (t) {
    case QR_Q4_0: case QR_Q4_1: case QR_Q5_0: case QR_Q5_1: case QR_Q6_0: return 32;
    case QR_Q4_K: case QR_Q5_K: case QR_Q6_K: return 256;
    case QR_Q8_K128: return 128;
    case QR_Q8_K64: return 64;
    case QR_Q8_K16: return 16;
    default: return 0;
  }
}

size_t block_bytes(int t) {
  switch (t) {
    case QR_Q4_0: return 20;
    case QR_Q4_1: return 24;
    case QR_Q5_0: return 24;
    case QR_Q5_1: return 28;
    case QR_Q4_K: return 144;
    case QR_Q8_K128: return 140;
    case QR_Q6_0: return 28;
    case QR_Q8_K64: return 72;
    case QR_Q8_K16: return 24;
    case QR_Q6_K: return 212;
    case QR_Q5_K: return 176;
    default: return 0;
  }
}

bool aligned16(const void* p) { return qr_aligned(p, 16); }


// Bytes of LDS of the workgroup that quantizes one row: the staged row and
// the cross-wave partial sums.
size_t row_lds_bytes(int n_per_row, bool bf16, int waves) {
  return (size_t)(n_per_row / QK) * (bf16 ? LDS_BF16_STRIDE * 2 : LDS_F32_STRIDE * 4) + 8 * (size_t)waves;
}

// Waves of the workgroup that quantizes one row of n_per_row values. Each
// lane solves groups tid, tid + 64W, ..., so any W works; W is chosen for
// the lanes kept busy and the waves a compute unit holds: at most 16 (four
// per SIMD, the register budget of the row kernels) and as many workgroups
// as its 160 KiB of LDS take. One wave per 64 groups, the plain choice,
// wins ties; another W must do better by more than a tenth. (Rows of 11008
// bf16 values, 344 groups: six waves give two workgroups, 12 waves, per CU;
// three waves over two passes give five, 15 waves.)
int row_waves(int n_per_row, bool bf16) {
  const int groups = n_per_row / QK;
  auto score = [&](int w) {
    const int lanes = WAVE * w;
    const int passes = (groups + lanes - 1) / lanes;
    const double busy = (double)groups / ((double)passes * lanes);
    int wgs = (int)(LDS_PER_WORKGROUP / row_lds_bytes(n_per_row, bf16, w));
    if (wgs > 16 / w) wgs = 16 / w;
    const int waves = wgs * w;
    return busy * (waves < 16 ? waves : 16);
  };
  int plain = (groups + WAVE - 1) / WAVE;
  if (plain > MAX_ROW_WAVES) plain = MAX_ROW_WAVES;
  int best = plain;
  double best_score = score(plain);
  for (int w = 1; w <= MAX_ROW_WAVES; ++w) {
    const double sc = score(w);
    if (sc > 1.1 * best_score) {
      best = w;
      best_score = sc;
    }
  }
  return best;
}

// Rows per block of the streaming row kernel for this width, or 0 when the
// plain kernel is as good: the streaming layout must keep every lane busy
// where the plain one does not (same W, one wave per 64 groups), hold as many
// waves per compute unit with its two row slots of LDS, and meet the
// kernel's conditions (a pass spans at most two rows; each pass needs at
// most one row more than the one before).
int stream_block_rows(int n_per_row, bool bf16) {
  const int groups = n_per_row / QK;
  int w = (groups + WAVE - 1) / WAVE;
  if (w > MAX_ROW_WAVES) return 0;
  const int lanes = WAVE * w;
  if (groups % lanes == 0 || groups % 8 != 0) return 0;
  int a = groups, b = lanes;   // gcd
  while (b) { const int t = a % b; a = b; b = t; }
  const int block_rows = lanes / a;
  const int passes = block_rows * groups / lanes;
  int64_t prev_last = 0;
  for (int p = 0; p < passes; ++p) {
    const int64_t first = (int64_t)p * lanes / groups;
    const int64_t last = ((int64_t)p * lanes + lanes - 1) / groups;
    if (last - first > 1 || last - prev_last > 1) return 0;
    prev_last = last;
  }
  const size_t lds = 2 * (row_lds_bytes(n_per_row, bf16, w) - 8 * (size_t)w) + 8 * (size_t)w;
  int wgs = (int)(LDS_PER_WORKGROUP / lds);
  if (wgs > 16 / w) wgs = 16 / w;
  const int waves = wgs * w < 16 ? wgs * w : 16;
  // the plain kernel's best choice, scored the same way as row_waves does
  const int pw = row_waves(n_per_row, bf16);
  const int plane = WAVE * pw;
  const int ppasses = (groups + plane - 1) / plane;
  const double pbusy = (double)groups / ((double)ppasses * plane);
  int pwgs = (int)(LDS_PER_WORKGROUP / row_lds_bytes(n_per_row, bf16, pw));
  if (pwgs > 16 / pw) pwgs = 16 / pw;
  const int pwaves = pwgs * pw < 16 ? pwgs * pw : 16;
  return (double)waves > 1.05 * pbusy * pwaves ? block_rows : 0;
}

// Raises a row kernel's dynamic-LDS limit to the whole 160 KiB once per
// device and kernel (each instantiation has its own flags), for workgroups
// that need more than 64 KiB. The attribute is set on the current device, so
// for a stream of another device that device is made current for the call.
// The flags may be read and set by several host threads at once.
template <int TYPE, bool BF16, bool VAR, bool STREAM>
int raise_lds_limit(const void* kern, size_t lds, hipStream_t stream) {
  constexpr int MAX_DEVICES = 64;
  static std::atomic<bool> attr_set[MAX_DEVICES];
  if (lds <= 65536) return QR_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipGetDevice failed");
  int sdev = dev;
  if (stream && hipStreamGetDevice(stream, &sdev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipStreamGetDevice failed");
  if (sdev < 0 || sdev >= MAX_DEVICES || !attr_set[sdev].load(std::memory_order_acquire)) {
    if (sdev != dev && hipSetDevice(sdev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipSetDevice failed");
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_PER_WORKGROUP);
    if (sdev != dev && hipSetDevice(dev) != hipSuccess) return qr_fail(QR_EDEVICE, "hipSetDevice failed");
    if (e != hipSuccess) return qr_fail(QR_EDEVICE, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    if (sdev >= 0 && sdev < MAX_DEVICES) attr_set[sdev].store(true, std::memory_order_release);
  }
  return QR_OK;
}

template <int TYPE, bool BF16, bool VAR>
int launch_rows(const void* x, const float* imatrix, int64_t n_rows, int n_per_row, int64_t rows_per_group,
                void* out, size_t row_bytes, int weighting, int fit, hipStream_t stream) {
  const int block_rows = stream_block_rows(n_per_row, BF16);
  if (block_rows > 0) {
    auto kern = k_quantize_rows_stream<TYPE, BF16, VAR>;
    const int waves = (n_per_row / QK + WAVE - 1) / WAVE;
    const size_t lds = 2 * (row_lds_bytes(n_per_row, BF16, waves) - 8 * (size_t)waves) + 8 * (size_t)waves;
    const int rc = raise_lds_limit<TYPE, BF16, VAR, true>(reinterpret_cast<const void*>(kern), lds, stream);
    if (rc != QR_OK) return rc;
    const int64_t blocks = (n_rows + block_rows - 1) / block_rows;
    hipLaunchKernelGGL(kern, dim3((uint32_t)blocks), dim3(WAVE * waves), lds, stream, x, imatrix, n_per_row, n_rows,
                       rows_per_group, reinterpret_cast<uint8_t*>(out), (int64_t)row_bytes, weighting, fit,
                       block_rows);
    return qr_check_launch("k_quantize_rows_stream");
  }
  auto kern = k_quantize_rows<TYPE, BF16, VAR>;
  const int waves = row_waves(n_per_row, BF16);
  const size_t lds = row_lds_bytes(n_per_row, BF16, waves);
  const int rc = raise_lds_limit<TYPE, BF16, VAR, false>(reinterpret_cast<const void*>(kern), lds, stream);
  if (rc != QR_OK) return rc;
  hipLaunchKernelGGL(kern, dim3((uint32_t)n_rows), dim3(WAVE * waves), lds, stream, x, imatrix, n_per_row,
                     rows_per_group, reinterpret_cast<uint8_t*>(out), (int64_t)row_bytes, weighting, fit);
  return qr_check_launch("k_quantize_rows");
}

template <bool BF16, bool VAR>
int dispatch_rows(int t, const void* x, const float* imatrix, int64_t n_rows, int n_per_row,
                  int64_t rows_per_group, void* out, size_t row_bytes, int weighting, int fit, hipStream_t s) {
#define QR_ROWS_LAUNCH(T) \
  launch_rows<T, BF16, VAR>(x, imatrix, n_rows, n_per_row, rows_per_group, out, row_bytes, weighting, fit, s)
  switch (t) {
    case QR_Q4_0: return QR_ROWS_LAUNCH(QR_Q4_0);
    case QR_Q4_1: return QR_ROWS_LAUNCH(QR_Q4_1);
    case QR_Q5_0: return QR_ROWS_LAUNCH(QR_Q5_0);
    case QR_Q5_1: return QR_ROWS_LAUNCH(QR_Q5_1);
    case QR_Q4_K: return QR_ROWS_LAUNCH(QR_Q4_K);
    case QR_Q6_0: return QR_ROWS_LAUNCH(QR_Q6_0);
    case QR_Q6_K: return QR_ROWS_LAUNCH(QR_Q6_K);
    case QR_Q5_K: return QR_ROWS_LAUNCH(QR_Q5_K);
    default: return qr_fail(QR_EINVAL_TYPE, "type %d is not a weight-row type", t);
  }
#undef QR_ROWS_LAUNCH
}

// Validation and launch shared by the row quantizers. The pages' weighting
// with the default sub-scales runs in the kernels compiled for it alone;
// every other choice in the variants.
int quantize_rows_common(int t, int src, const void* x, const float* imatrix, int64_t n_groups,
                         int64_t rows_per_group, int64_t n_per_row, int weighting, int fit, void* out,
                         void* stream) {
  if (!qr_is_weight_type(t)) return qr_fail(QR_EINVAL_TYPE, "type %d is not a weight-row type", t);
  if (src != QR_F32 && src != QR_BF16) return qr_fail(QR_EINVAL_TYPE, "source dtype %d is not f32/bf16", src);
  if (weighting < QR_W_SQRT_SIGMA2_X2 || weighting > QR_W_IMATRIX_ONLY)
    return qr_fail(QR_EINVAL_TYPE, "weighting %d is not a qr_weighting", weighting);
  if (fit != QR_FIT_MAX && fit != QR_FIT_WEIGHTED)
    return qr_fail(QR_EINVAL_TYPE, "subscale_fit %d is not a qr_subscale_fit", fit);
  if (n_groups < 0 || rows_per_group < 0) return qr_fail(QR_EINVAL_SHAPE, "negative row count");
  const int be = block_elems(t);
  const int64_t max_row = src == QR_F32 ? QR_MAX_ROW_F32 : QR_MAX_ROW_BF16;
  if (n_per_row <= 0 || n_per_row % be != 0 || n_per_row > max_row)
    return qr_fail(QR_EINVAL_SHAPE, "n_per_row=%lld must be a positive multiple of %d and at most %lld",
                (long long)n_per_row, be, (long long)max_row);
  if (rows_per_group != 0 && n_groups > INT64_MAX / rows_per_group)
    return qr_fail(QR_EOVERFLOW, "n_groups * rows_per_group overflows");
  const int64_t n_rows = n_groups * rows_per_group;
  if (n_rows == 0) return QR_OK;
  if (n_rows > (int64_t)UINT32_MAX) return qr_fail(QR_EOVERFLOW, "n_rows=%lld exceeds 2^32-1", (long long)n_rows);
  // one workgroup per row: the launch's work items must stay below 2^32
  const int64_t row_threads = (int64_t)WAVE * row_waves((int)n_per_row, src == QR_BF16);
  if (n_rows > (int64_t)UINT32_MAX / row_threads)
    return qr_fail(QR_EINVAL_SHAPE, "n_rows=%lld rows of %d threads exceed one launch (at most %lld rows)",
                   (long long)n_rows, (int)row_threads, (long long)((int64_t)UINT32_MAX / row_threads));
  const size_t rb = qr_row_bytes(t, n_per_row);
  if ((uint64_t)n_rows > SIZE_MAX / rb || (uint64_t)n_rows > SIZE_MAX / ((uint64_t)n_per_row * 4))
    return qr_fail(QR_EOVERFLOW, "buffer size overflows");
  if (!x || !out) return qr_fail(QR_EINVAL_PTR, "x and out must be non-NULL");
  if (!aligned16(x) || !aligned16(out) || (imatrix && !aligned16(imatrix)))
    return qr_fail(QR_EINVAL_PTR, "device pointers must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int n = (int)n_per_row;
  if (t != QR_Q4_K && t != QR_Q5_K) fit = QR_FIT_MAX;   // no 6-bit sub-scales to fit
  if (weighting == QR_W_SQRT_SIGMA2_X2 && fit == QR_FIT_MAX)
    return src == QR_F32 ? dispatch_rows<false, false>(t, x, imatrix, n_rows, n, rows_per_group, out, rb, 0, 0, s)
                         : dispatch_rows<true, false>(t, x, imatrix, n_rows, n, rows_per_group, out, rb, 0, 0, s);
  return src == QR_F32
             ? dispatch_rows<false, true>(t, x, imatrix, n_rows, n, rows_per_group, out, rb, weighting, fit, s)
             : dispatch_rows<true, true>(t, x, imatrix, n_rows, n, rows_per_group, out, rb, weighting, fit, s);
}

int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  const int64_t cap = 1 << 17;    // plenty of waves in flight for the streaming kernels
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

static thread_local char g_err[512];

void qr_clear_error() { g_err[0] = 0; }

int qr_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int qr_check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return qr_fail(QR_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return QR_OK;
}

extern "C" {

const char* qr_last_error(void) { return g_err; }

int qr_block_elems(int t) { return block_elems(t); }

size_t qr_row_bytes(int t, int64_t n_per_row) {
  const int be = block_elems(t);
  if (be == 0 || n_per_row < 0 || n_per_row % be != 0) return 0;
  return (size_t)(n_per_row / be) * block_bytes(t);
}

void qr_solver_constants(int32_t* c) {
  c[0] = (int32_t)(CAND_STEP * 4.0f);
  c[1] = SYM_CAND;
  c[2] = SYM_FLIP_PASSES;
  c[3] = ASYM_CAND;
  c[4] = ASYM_FLIP_PASSES;
  c[5] = QK;
}

int qr_quantize_rows_grouped(int t, int src, const void* x, const float* imatrix, int64_t n_groups,
                             int64_t rows_per_group, int64_t n_per_row, void* out, void* stream) {
  qr_clear_error();
  return quantize_rows_common(t, src, x, imatrix, n_groups, rows_per_group, n_per_row, QR_W_SQRT_SIGMA2_X2,
                              QR_FIT_MAX, out, stream);
}

int qr_quantize_rows_ex(int t, int src, const void* x, const float* imatrix, int64_t n_groups,
                        int64_t rows_per_group, int64_t n_per_row, int weighting, int subscale_fit, void* out,
                        void* stream) {
  qr_clear_error();
  return quantize_rows_common(t, src, x, imatrix, n_groups, rows_per_group, n_per_row, weighting, subscale_fit,
                              out, stream);
}

int qr_quantize_rows_weighted(int t, int src, const void* x, const float* imatrix, int64_t n_rows,
                              int64_t n_per_row, int weighting, void* out, void* stream) {
  qr_clear_error();
  if (n_rows < 0) return qr_fail(QR_EINVAL_SHAPE, "negative row count");
  return quantize_rows_common(t, src, x, imatrix, 1, n_rows, n_per_row, weighting, QR_FIT_MAX, out, stream);
}

int qr_quantize_rows(int t, int src, const void* x, const float* imatrix, int64_t n_rows, int64_t n_per_row,
                     void* out, void* stream) {
  if (n_rows < 0) {
    qr_clear_error();
    return qr_fail(QR_EINVAL_SHAPE, "negative row count");
  }
  return qr_quantize_rows_grouped(t, src, x, imatrix, 1, n_rows, n_per_row, out, stream);
}

int qr_quantize_activations_q8k(int t, int src, const void* x, int64_t n_rows, int64_t n_per_row, void* out,
                                void* stream) {
  qr_clear_error();
  if (t != QR_Q8_K128 && t != QR_Q8_K64 && t != QR_Q8_K16)
    return qr_fail(QR_EINVAL_TYPE, "type %d is not a Q8_K activation type", t);
  if (src != QR_F32 && src != QR_BF16) return qr_fail(QR_EINVAL_TYPE, "source dtype %d is not f32/bf16", src);
  const int B = block_elems(t);
  if (n_rows < 0 || n_per_row <= 0 || n_per_row % B != 0)
    return qr_fail(QR_EINVAL_SHAPE, "n_per_row=%lld must be a positive multiple of %d", (long long)n_per_row, B);
  if (n_rows == 0) return QR_OK;
  if (n_per_row / B > INT32_MAX) return qr_fail(QR_EOVERFLOW, "row too long");
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / ((uint64_t)n_per_row * 4)) return qr_fail(QR_EOVERFLOW, "size overflows");
  if (!x || !out) return qr_fail(QR_EINVAL_PTR, "x and out must be non-NULL");
  if (!aligned16(x) || !aligned16(out)) return qr_fail(QR_EINVAL_PTR, "device pointers must be 16-byte aligned");
  const int64_t n_blocks = n_rows * (n_per_row / B);
  const int64_t chunks = (n_blocks + q8_chunk_blocks(B) - 1) / q8_chunk_blocks(B);
  const int grid = grid_for(chunks, 4);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* o = reinterpret_cast<uint8_t*>(out);
  const bool bf = src == QR_BF16;
  switch (B) {
    case 128:
      if (bf) hipLaunchKernelGGL((k_quantize_q8k<128, true>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      else hipLaunchKernelGGL((k_quantize_q8k<128, false>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      break;
    case 64:
      if (bf) hipLaunchKernelGGL((k_quantize_q8k<64, true>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      else hipLaunchKernelGGL((k_quantize_q8k<64, false>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      break;
    default:
      if (bf) hipLaunchKernelGGL((k_quantize_q8k<16, true>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      else hipLaunchKernelGGL((k_quantize_q8k<16, false>), dim3(grid), dim3(256), 0, s, x, n_blocks, o);
      break;
  }
  return qr_check_launch("k_quantize_q8k");
}

int qr_quantize_activations_q8k128(int src, const void* x, int64_t n_rows, int64_t n_per_row, void* out,
                                   void* stream) {
  return qr_quantize_activations_q8k(QR_Q8_K128, src, x, n_rows, n_per_row, out, stream);
}

int qr_dequantize_rows(int t, const void* in, int64_t n_rows, int64_t n_per_row, float* out, void* stream) {
  qr_clear_error();
  const int be = block_elems(t);
  if (be == 0) return qr_fail(QR_EINVAL_TYPE, "unknown type %d", t);
  if (n_rows < 0 || n_per_row <= 0 || n_per_row % be != 0)
    return qr_fail(QR_EINVAL_SHAPE, "n_per_row=%lld must be a positive multiple of %d", (long long)n_per_row, be);
  if (n_rows == 0) return QR_OK;
  if (n_per_row > INT32_MAX) return qr_fail(QR_EOVERFLOW, "row too long");
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / ((uint64_t)n_per_row * 4)) return qr_fail(QR_EOVERFLOW, "size overflows");
  if (!in || !out) return qr_fail(QR_EINVAL_PTR, "in and out must be non-NULL");
  if (!aligned16(in) || !aligned16(out)) return qr_fail(QR_EINVAL_PTR, "device pointers must be 16-byte aligned");
  const int64_t n_items = n_rows * n_per_row / 4;
  const int grid = grid_for((n_items + DQ_STEPS - 1) / DQ_STEPS, 256);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* p = reinterpret_cast<const uint8_t*>(in);
  switch (t) {
    case QR_Q4_0: hipLaunchKernelGGL(k_dequantize<QR_Q4_0>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q4_1: hipLaunchKernelGGL(k_dequantize<QR_Q4_1>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q5_0: hipLaunchKernelGGL(k_dequantize<QR_Q5_0>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q5_1: hipLaunchKernelGGL(k_dequantize<QR_Q5_1>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q4_K: hipLaunchKernelGGL(k_dequantize<QR_Q4_K>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q6_0: hipLaunchKernelGGL(k_dequantize<QR_Q6_0>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q6_K: hipLaunchKernelGGL(k_dequantize<QR_Q6_K>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q5_K: hipLaunchKernelGGL(k_dequantize<QR_Q5_K>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q8_K64: hipLaunchKernelGGL(k_dequantize<QR_Q8_K64>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    case QR_Q8_K16: hipLaunchKernelGGL(k_dequantize<QR_Q8_K16>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
    default: hipLaunchKernelGGL(k_dequantize<QR_Q8_K128>, dim3(grid), dim3(256), 0, s, p, n_items, out); break;
  }
  return qr_check_launch("k_dequantize");
}

}  // extern "C"
