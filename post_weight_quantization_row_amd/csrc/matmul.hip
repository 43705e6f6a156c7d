// matmul.hip -- gfx950 kernel and C-ABI of the product of quantized weight
// rows with Q8_K activation rows of 128, 64 or 16 values per block
// (declared in qrow_matmul.h).
//
// Following this page (cited by title and section):
//  [Q8] "ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …", sections
//       修复前的数值隐患 and 修复方案: integer products of weight and activation
//       codes, the weight offset removed with the activation code sums, which
//       Q8_K_128 keeps as unscaled int16 per 32 codes; section 技术启示与后续演进
//       for the 64- and 16-value members of the family.
//
// Execution model (gfx950, wave64). A workgroup of four waves owns a few
// weight rows and a tile of TT tokens. With TT > 1 the tile's activation
// rows (one contiguous range) are unpacked once into LDS (codes, fp32
// scales, code sums), 16 bytes per load where aligned; with one token each
// lane reads its groups' activation words from the packed row (L2-resident)
// together with the weights. L lanes own a row (64 for one token, 32 for a
// tile); lane s takes the row's 32-weight groups s, s + L, ..., loads their
// packed bytes unconditionally so that a batch is in flight at once
// (consecutive lanes read consecutive blocks), expands the 4-bit codes (and
// the fifth bit) into bytes, and for every token forms sum(u*q) with eight
// v_dot4 instructions, folds the offset with the int16 code sum, and adds
// the scaled term in fp32. A butterfly over the row's lanes gives its
// outputs. One token is bound by reading the weights from HBM; tiles of
// tokens by instruction issue (eight v_dot4 plus about thirty addressing,
// LDS and scaling instructions per 32 weights and token). With 16-value
// activation blocks a weight group spans two activation scales: the two
// halves of the dot product are scaled and added separately.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qr_internal.h"
#include "qrow.h"
#include "qrow_matmul.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int MMQ_WAVES = 4;
constexpr int MMQ_THREADS = WAVE * MMQ_WAVES;
// Lanes per weight row and groups per lane per batch: one token (a decode
// step) gives each row a whole wave, one group at a time; a tile of tokens
// gives each row half a wave, two groups at a time (measured best of 16/32/64
// lanes x 1/2/4 groups).
__host__ __device__ constexpr int mmq_lanes(int tt) { return tt == 1 ? 64 : 32; }
__host__ __device__ constexpr int mmq_batch(int tt) { return tt == 1 ? 1 : 2; }
__host__ __device__ constexpr int mmq_rows(int tt) { return MMQ_THREADS / mmq_lanes(tt); }
constexpr int MMQ_LDS_BUDGET = 64 * 1024;         // bytes of staged activations

// Activation formats: values per block, words per packed block, values per
// code sum (Q8_K128: 140 B, Q8_K64: 72 B, Q8_K16: 24 B with a zero pad).
__host__ __device__ constexpr int act_block(int act) { return act == QR_Q8_K128 ? 128 : act == QR_Q8_K64 ? 64 : 16; }
__host__ __device__ constexpr int act_words(int act) { return act == QR_Q8_K128 ? 35 : act == QR_Q8_K64 ? 18 : 6; }
__host__ __device__ constexpr int act_sum_unit(int act) { return act == QR_Q8_K16 ? 16 : 32; }

// LDS bytes for a tile of tt tokens of n_in values: codes, scales, sums.
__host__ __device__ constexpr int64_t mmq_lds_bytes(int tt, int64_t n_in, int act) {
  return (int64_t)tt * (n_in + n_in / act_block(act) * 4 + n_in / act_sum_unit(act) * 4);
}

// Four 2-bit fields of b (bits 2e, 2e+1) spread to bits 8e, 8e+1.
__device__ __forceinline__ uint32_t spread2(uint32_t b) {
  return (b & 3u) | ((b & 0x0cu) << 6) | ((b & 0x30u) << 12) | ((b & 0xc0u) << 18);
}

// 4 bits t (0..15) spread into bit 0 of each byte: bit k -> bit 8k.
__device__ __forceinline__ uint32_t spread4(uint32_t t) { return (t * 0x00204081u) & 0x01010101u; }

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ float half_bits(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// One 32-weight group of a row, ready for the token loop: the codes as
// bytes (lo: elements 0..15, hi: 16..31) and the float parts of the decode.
struct Group {
  uint32_t lo[4], hi[4];
  float sa;  // scale part:  d (legacy), d*sc (Q4_K, Q5_K), d*s of the first 16 (Q6_K)
  float sb;  // offset part: the level offset 8/16 (symmetric), m (Q4_1/Q5_1) or dmin*mn (Q4_K, Q5_K)
  float sa1; // Q6_K: d*s of the second 16 (its codes are signed levels, no offset)
};

// The packed bytes of one group as loaded (up to nine words), kept apart
// from the decoding so that a batch of loads can be in flight at once.
struct RawGroup {
  uint32_t v[9];
};

template <int TYPE>
__device__ __forceinline__ RawGroup load_raw(const uint8_t* __restrict__ row, int g) {
  RawGroup R;
  if (TYPE == QR_Q6_K) {
    // d | the sub-scale word | 16 nibble bytes | the 8-byte plane (212-byte
    // blocks are only 4-byte aligned)
    const uint8_t* sb = row + (int64_t)(g >> 3) * 212;
    const int j = g & 7;
    R.v[0] = ld32(sb);
    R.v[1] = ld32(sb + 4 + 4 * (j >> 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) R.v[2 + k] = ld32(sb + 20 + 16 * j + 4 * k);
    R.v[6] = ld32(sb + 148 + 8 * j);
    R.v[7] = ld32(sb + 152 + 8 * j);
  } else if (TYPE == QR_Q4_K || TYPE == QR_Q5_K) {
    // header | (Q5_K: the group's fifth-bit word) | its 16 nibble bytes
    constexpr bool Q5 = TYPE == QR_Q5_K;
    const uint8_t* sb = row + (int64_t)(g >> 3) * (Q5 ? 176 : 144);
    const u32x4 h = *reinterpret_cast<const u32x4*>(sb);
    const u32x4 c = *reinterpret_cast<const u32x4*>(sb + (Q5 ? 48 : 16) + 16 * (g & 7));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      R.v[k] = h[k];
      R.v[4 + k] = c[k];
    }
    if (Q5) R.v[8] = ld32(sb + 16 + 4 * (g & 7));
  } else {
    constexpr int WORDS = TYPE == QR_Q4_0 ? 5 : (TYPE == QR_Q5_1 || TYPE == QR_Q6_0) ? 7 : 6;
    const uint8_t* p = row + (int64_t)g * (WORDS * 4);
#pragma unroll
    for (int k = 0; k < WORDS; ++k) R.v[k] = ld32(p + 4 * k);
  }
  return R;
}

// One token's activation words for one 32-value group of a packed
// activation row: the 8 code words, the word(s) holding its int16 code
// sum(s), the scale(s) (the second sum and scale only for 16-value blocks,
// whose two blocks cover the group's halves).
struct RawAct {
  uint32_t q[8];
  uint32_t sums, sums1;
  uint32_t d, d1;
};

template <int ACT>
__device__ __forceinline__ RawAct load_act(const uint8_t* __restrict__ xrow, int g) {
  RawAct A;
  if constexpr (ACT == QR_Q8_K16) {
    const uint8_t* b0 = xrow + (int64_t)g * 48;
    const uint8_t* b1 = b0 + 24;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      A.q[c] = ld32(b0 + 4 + 4 * c);
      A.q[4 + c] = ld32(b1 + 4 + 4 * c);
    }
    A.sums = ld32(b0 + 20);
    A.sums1 = ld32(b1 + 20);
    A.d = ld32(b0);
    A.d1 = ld32(b1);
  } else {
    constexpr int PER = act_block(ACT) / 32;           // groups per block
    const uint8_t* blk = xrow + (int64_t)(g / PER) * (act_words(ACT) * 4);
    const int gi = g & (PER - 1);
#pragma unroll
    for (int c = 0; c < 8; ++c) A.q[c] = ld32(blk + 4 + 32 * gi + 4 * c);
    A.sums = ld32(blk + 4 + act_block(ACT) + 4 * (gi >> 1));
    A.d = ld32(blk);
    A.sums1 = 0;
    A.d1 = 0;
  }
  return A;
}

template <int TYPE>
__device__ __forceinline__ Group unpack(const RawGroup& R, int g) {
  Group G;
  G.sa1 = 0.0f;
  if (TYPE == QR_Q6_K) {
    // codes u = nibble | plane bits << 4, turned into signed levels u - 32:
    // per byte, x = u ^ 32 sign-extended from bit 5
    const int j = g & 7;
    const float dA = half_bits(R.v[0]);
    const uint32_t sw = R.v[1] >> (16 * (j & 1));
    G.sa = dA * (float)(int)(int8_t)(uint8_t)(sw & 255u);
    G.sa1 = dA * (float)(int)(int8_t)(uint8_t)((sw >> 8) & 255u);
    G.sb = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t wk = R.v[2 + k];
      const uint32_t lo = (wk & 0x0f0f0f0fu) | (spread2((R.v[6] >> (8 * k)) & 255u) << 4);
      const uint32_t hi = ((wk >> 4) & 0x0f0f0f0fu) | (spread2((R.v[7] >> (8 * k)) & 255u) << 4);
      const uint32_t xl = lo ^ 0x20202020u, xh = hi ^ 0x20202020u;
      G.lo[k] = xl | ((xl & 0x20202020u) * 6u);
      G.hi[k] = xh | ((xh & 0x20202020u) * 6u);
    }
    return G;
  }
  uint32_t qh = 0;
  int qs0;  // first word of the 16 code bytes
  if (TYPE == QR_Q4_K || TYPE == QR_Q5_K) {
    const int j = g & 7;
    const uint32_t h1 = R.v[1], h2 = R.v[2], h3 = R.v[3];
    const uint64_t sc6 = (uint64_t)h1 | ((uint64_t)(h2 & 0xffffu) << 32);
    const uint64_t mn6 = (uint64_t)(h2 >> 16) | ((uint64_t)h3 << 16);
    const float d = half_bits(R.v[0]), dmin = half_bits(R.v[0] >> 16);
    G.sa = d * (float)((sc6 >> (6 * j)) & 63);     // exact: 11-bit times 6-bit
    G.sb = dmin * (float)((mn6 >> (6 * j)) & 63);
    if (TYPE == QR_Q5_K) qh = R.v[8];
    qs0 = 4;
  } else if (TYPE == QR_Q6_0) {
    G.sa = __builtin_bit_cast(float, R.v[0]);
    G.sb = 32.0f;
    qs0 = 3;
  } else {
    G.sa = __builtin_bit_cast(float, R.v[0]);
    if (TYPE == QR_Q4_1 || TYPE == QR_Q5_1) G.sb = __builtin_bit_cast(float, R.v[1]);
    else G.sb = TYPE == QR_Q4_0 ? 8.0f : 16.0f;
    if (TYPE == QR_Q5_0) qh = R.v[1];
    if (TYPE == QR_Q5_1) qh = R.v[2];
    qs0 = TYPE == QR_Q4_0 ? 1 : TYPE == QR_Q5_1 ? 3 : 2;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t wk = R.v[qs0 + k];
    G.lo[k] = wk & 0x0f0f0f0fu;
    G.hi[k] = (wk >> 4) & 0x0f0f0f0fu;
    if (TYPE == QR_Q5_0 || TYPE == QR_Q5_1 || TYPE == QR_Q5_K) {
      G.lo[k] |= spread4((qh >> (4 * k)) & 15u) << 4;
      G.hi[k] |= spread4((qh >> (16 + 4 * k)) & 15u) << 4;
    }
    if (TYPE == QR_Q6_0) {  // bits 4, 5 from the 2-bit plane (byte k of each half)
      G.lo[k] |= spread2((R.v[1] >> (8 * k)) & 255u) << 4;
      G.hi[k] |= spread2((R.v[2] >> (8 * k)) & 255u) << 4;
    }
  }
  return G;
}

// The scaled term of one activation block's share of a group: I = sum(u*q)
// over that share, bs its code sum, da its scale.
template <int TYPE>
__device__ __forceinline__ float add_term(const Group& G, int I, int bs, float da, float acc) {
  if (TYPE == QR_Q4_0 || TYPE == QR_Q5_0 || TYPE == QR_Q6_0) {
    // d * (sum(u*q) - offset * bsum), exact in int32
    const int J = I - (TYPE == QR_Q4_0 ? 8 : TYPE == QR_Q5_0 ? 16 : 32) * bs;
    return __builtin_fmaf(G.sa * da, (float)J, acc);
  } else if (TYPE == QR_Q4_1 || TYPE == QR_Q5_1) {
    // d * sum(u*q) + m * bsum
    return __builtin_fmaf(da, __builtin_fmaf(G.sa, (float)I, G.sb * (float)bs), acc);
  } else {
    // d*sc * sum(u*q) - dmin*mn * bsum
    return __builtin_fmaf(da, __builtin_fmaf(G.sa, (float)I, -(G.sb * (float)bs)), acc);
  }
}

template <int TYPE, int ACT, int TT>
__global__ __launch_bounds__(MMQ_THREADS) void k_matmul_q8k(const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ x, int64_t n_out,
                                                            int64_t n_tok, int n_in, int64_t w_row_bytes,
                                                            float* __restrict__ y) {
  constexpr int AB = act_block(ACT);          // values per activation block
  constexpr int AW = act_words(ACT);          // words per packed activation block
  constexpr int CW = AB / 4;                  // code words per activation block
  constexpr bool SPLIT = ACT == QR_Q8_K16;    // two activation blocks per group
  extern __shared__ uint32_t lds[];
  const int nb = n_in / AB;   // activation blocks per row
  const int ng = n_in / 32;   // 32-value groups per row
  // Block-major over the tile (block tb = t * nb + b): code words
  // [TT * nb][CW] (that is, [TT * ng][8]), scales [TT * nb], code sums
  // [TT * n_in / sum unit].
  uint32_t* lq = lds;
  float* ld = reinterpret_cast<float*>(lds + TT * nb * CW);
  int32_t* lsum = reinterpret_cast<int32_t*>(ld + TT * nb);

  // L lanes own one row; lane s takes the row's groups s, s + L, ..., NF at
  // a time, the next batch requested before the current one is used.
  constexpr int L = mmq_lanes(TT);
  constexpr int NF = mmq_batch(TT);
  constexpr int STEP = L * NF;
  const int sub = threadIdx.x & (L - 1);
  const int64_t r = (int64_t)blockIdx.x * mmq_rows(TT) + threadIdx.x / L;
  const bool row_ok = r < n_out;
  const uint8_t* row = w + (row_ok ? r : 0) * w_row_bytes;
  const int64_t t0 = (int64_t)blockIdx.y * TT;
  const uint8_t* xt = x + t0 * (int64_t)nb * AW * 4;
  RawGroup cur[NF], nxt[NF];
  RawAct acur[TT == 1 ? NF : 1], anxt[TT == 1 ? NF : 1];
  auto load_batch = [&](RawGroup (&b)[NF], RawAct (&ab)[TT == 1 ? NF : 1], int g0) {
    // unconditional loads (past the end: the row's last group, unused), so
    // that the whole batch is issued back to back; with one token the
    // group's activation words come with it
#pragma unroll
    for (int u = 0; u < NF; ++u) {
      const int g = g0 + u * L;
      const int gc = g < ng ? g : ng - 1;
      b[u] = load_raw<TYPE>(row, gc);
      if (TT == 1) ab[TT == 1 ? u : 0] = load_act<ACT>(xt, gc);
    }
  };
  if (TT > 1) {
    // The tile's activation rows are contiguous: stage them with eight
    // independent loads in flight per thread (absent tokens read as 0),
    // 16 bytes at a time when the rows are whole 16-byte vectors.
    const int total = TT * nb * AW;
    const int64_t tok_left = n_tok - t0;
    const int valid = tok_left >= TT ? total : (int)tok_left * nb * AW;
    auto put = [&](int idx, uint32_t v) {
      const int tb = idx / AW;
      const int k = idx - tb * AW;
      if (k == 0) {
        ld[tb] = __builtin_bit_cast(float, v);
      } else if (k <= CW) {
        lq[tb * CW + (k - 1)] = v;
      } else if (SPLIT) {
        lsum[tb] = (int32_t)(int16_t)(v & 0xffffu);  // the upper half is the pad
      } else {
        const int g = tb * (AB / 32) + (k - 1 - CW) * 2;
        lsum[g] = (int32_t)(int16_t)(v & 0xffffu);
        lsum[g + 1] = (int32_t)(int16_t)(v >> 16);
      }
    };
    if ((nb * AW) % 4 == 0) {
      const int chunks = total / 4, valid4 = valid / 4;
      for (int base = threadIdx.x; base < chunks; base += MMQ_THREADS * 8) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = base + j * MMQ_THREADS;
          v[j] = *reinterpret_cast<const u32x4*>(xt + (int64_t)(c < valid4 ? c : valid4 - 1) * 16);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = base + j * MMQ_THREADS;
          if (c < chunks) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t ve = v[j][e];
              put(4 * c + e, c < valid4 ? ve : 0u);
            }
          }
        }
      }
    } else {
      for (int base = threadIdx.x; base < total; base += MMQ_THREADS * 8) {
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int idx = base + j * MMQ_THREADS;
          v[j] = ld32(xt + (int64_t)(idx < valid ? idx : valid - 1) * 4);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int idx = base + j * MMQ_THREADS;
          if (idx < total) put(idx, idx < valid ? v[j] : 0u);
        }
      }
    }
  }
  load_batch(cur, acur, sub);
  if (TT > 1) __syncthreads();

  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  for (int g0 = sub; g0 < ng && row_ok; g0 += STEP) {
    if (g0 + STEP < ng) load_batch(nxt, anxt, g0 + STEP);
#pragma unroll
    for (int u = 0; u < NF; ++u) {
      const int g = g0 + u * L;
      if (g >= ng) break;
      const Group G = unpack<TYPE>(cur[u], g);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int tg = t * ng + g;  // group index within the tile
        uint32_t a[8];
        int bs, bs1 = 0;
        float da, da1 = 0.0f;
        if (TT > 1) {
          const u32x4* qa = reinterpret_cast<const u32x4*>(lq + tg * 8);
          const u32x4 a0 = qa[0], a1 = qa[1];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            a[c] = a0[c];
            a[4 + c] = a1[c];
          }
          if (SPLIT) {
            bs = lsum[2 * tg];
            bs1 = lsum[2 * tg + 1];
            da = ld[2 * tg];
            da1 = ld[2 * tg + 1];
          } else {
            bs = lsum[tg];
            da = ld[tg / (AB / 32)];
          }
        } else {
          // one token: the words loaded with the group
          const RawAct& A = acur[TT == 1 ? u : 0];
#pragma unroll
          for (int c = 0; c < 8; ++c) a[c] = A.q[c];
          if (SPLIT) {
            bs = (int)(int16_t)(A.sums & 0xffffu);
            bs1 = (int)(int16_t)(A.sums1 & 0xffffu);
            da = __builtin_bit_cast(float, A.d);
            da1 = __builtin_bit_cast(float, A.d1);
          } else {
            bs = (int)(int16_t)((g & 1) ? (A.sums >> 16) : (A.sums & 0xffffu));
            da = __builtin_bit_cast(float, A.d);
          }
        }
        int ilo = 0, ihi = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) ilo = __builtin_amdgcn_sdot4((int)G.lo[c], (int)a[c], ilo, false);
        if (TYPE == QR_Q6_K) {
          // signed levels: sum(l*q) per 16-weight half, each with its scale
#pragma unroll
          for (int c = 0; c < 4; ++c) ihi = __builtin_amdgcn_sdot4((int)G.hi[c], (int)a[4 + c], ihi, false);
          acc[t] = __builtin_fmaf(G.sa * da, (float)ilo, acc[t]);
          acc[t] = __builtin_fmaf(G.sa1 * (SPLIT ? da1 : da), (float)ihi, acc[t]);
        } else if (SPLIT) {
#pragma unroll
          for (int c = 0; c < 4; ++c) ihi = __builtin_amdgcn_sdot4((int)G.hi[c], (int)a[4 + c], ihi, false);
          acc[t] = add_term<TYPE>(G, ilo, bs, da, acc[t]);
          acc[t] = add_term<TYPE>(G, ihi, bs1, da1, acc[t]);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) ilo = __builtin_amdgcn_sdot4((int)G.hi[c], (int)a[4 + c], ilo, false);
          acc[t] = add_term<TYPE>(G, ilo, bs, da, acc[t]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NF; ++u) cur[u] = nxt[u];
    if (TT == 1) {
#pragma unroll
      for (int u = 0; u < NF; ++u) acur[TT == 1 ? u : 0] = anxt[TT == 1 ? u : 0];
    }
  }
  // butterfly over the row's lanes: all of them end with the sums
#pragma unroll
  for (int t = 0; t < TT; ++t) {
#pragma unroll
    for (int m = L / 2; m >= 1; m >>= 1) acc[t] += __shfl_xor(acc[t], m, L);
  }
  if (row_ok && sub < TT && t0 + sub < n_tok) {
    float v = acc[0];
#pragma unroll
    for (int t = 1; t < TT; ++t)
      if (sub == t) v = acc[t];
    y[(t0 + sub) * n_out + r] = v;
  }
}

// -------------------------------------------------------------------------
// Many tokens: int8 matrix cores [Q8 修复方案: the same integer dot products
// and code-sum fold].
//
// With Q8_K_128 or Q8_K64 activations and at least MF_MIN_TOK tokens, a workgroup
// of four waves owns a tile of 64 tokens x 64 weight rows (x 32 rows when
// 64-row tiles would leave CUs without two workgroups). K advances one
// activation block (128 values, four 32-weight groups) per step:
//  * each thread decodes one (row, group) of the tile to 32 int8 codes in
//    LDS -- the symmetric types as signed levels, so that they need no
//    offset fold -- with its scale parts; the tile's activation blocks
//    (codes, scale, int16 code sums) are staged beside them. The global
//    loads for the next step are issued before this step's products.
//  * each wave owns 32 tokens x 32 (or 16) rows, 2 x 2 (or 2 x 1) tiles of
//    16 x 16: per group
//    one v_mfma_i32_16x16x32_i8 per tile (activations as A, weights as B)
//    gives the exact int32 dot products; they take the group's scale parts
//    with fp32 fused multiply-adds, and per activation block the sum takes
//    the activation scale and is added to a double accumulator. Q6_K's two
//    16-weight halves, each with its own scale, are two products with the
//    other half's codes zeroed.
// A block's sum has at most eight roundings, the accumulation is nearly
// exact and the result is rounded once: each output is within
// 2^-24 |y| + 8 * 2^-24 S of the exact product (S = sum of the terms'
// magnitudes), whatever n_in: inside the bound of the lane-parallel path.
//
// Output layout of the 16 x 16 x 32 product (checked on the device): lane l
// holds D[4 (l / 16) + v][l % 16], v = 0..3; A[i][k] and B[k][j] come from
// lane l with i or j = l % 16 and k = 8 (l / 16) + byte.

constexpr int MF_TOK = 64, MF_ROWS = 64, MF_THREADS = 256;
constexpr int MF_ROW_WORDS = 36;         // LDS words per token or row: 4 groups x 8 code words + 4 pad
// Fewer tokens: the lane-parallel kernel. Measured on the 11008x4096 Q4_K
// matrix: 51 against 51 us at 16 tokens, 50 against 70 at 24, 50 against 86
// at 32; at 8 tokens the lane-parallel kernel takes 11 us.
constexpr int MF_MIN_TOK = 17;
// Bytes of activations per 128-value step: one Q8_K_128 block (d, 128 codes,
// 4 int16 sums) or two Q8_K64 blocks (d, 64 codes, 2 int16 sums each).
__host__ __device__ constexpr int mf_step_bytes(int act) { return act == QR_Q8_K128 ? 140 : 144; }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// per byte: a code u in [0, 2 off) to the signed level u - off (off = 8, 16, 32)
template <int TYPE>
__device__ __forceinline__ uint32_t signed_levels(uint32_t u) {
  constexpr uint32_t OFF = TYPE == QR_Q4_0 ? 0x08080808u : TYPE == QR_Q5_0 ? 0x10101010u : 0x20202020u;
  constexpr uint32_t EXT = TYPE == QR_Q4_0 ? 0x1eu : TYPE == QR_Q5_0 ? 0x0eu : 0x06u;   // sign extension
  const uint32_t v = u ^ OFF;
  return v | ((v & OFF) * EXT);
}

// One K step of a tile in LDS. Rows of 36 words (word 8 g + k: code word k
// of group g) make the operand reads conflict free: the 16 tokens or rows of
// a product start 36 words apart, in distinct banks.
struct MfStage {
  uint32_t aq[MF_TOK][MF_ROW_WORDS];    // activation codes
  uint32_t wq[MF_ROWS][MF_ROW_WORDS];   // weight codes (symmetric types: signed levels)
  float wsa[4][MF_ROWS];                // scale part (Q6_K: of the first half)
  float wsb[4][MF_ROWS];                // offset part, signed (Q6_K: scale of the second half)
  float ad[2][MF_TOK];                  // activation scales (of each 64-value block for Q8_K64)
  float asum[4][MF_TOK];                // activation code sums per group (exact in fp32)
};

// RT row tiles of 16 per wave: tiles of 64 tokens x 64 rows (RT = 2), or
// x 32 rows (RT = 1) when the first would leave CUs without two workgroups.
// ACT: Q8_K_128 or Q8_K64 activations (a 64-value block holds two groups).
template <int TYPE, int ACT, int RT>
__global__ __launch_bounds__(MF_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void k_matmul_mfma(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ x, int64_t n_out, int64_t n_tok, int n_in,
    int64_t w_row_bytes, float* __restrict__ y) {
  constexpr bool SYM = TYPE == QR_Q4_0 || TYPE == QR_Q5_0 || TYPE == QR_Q6_0;
  constexpr bool Q6K = TYPE == QR_Q6_K;
  constexpr int ROWS = 32 * RT;   // rows of the tile
  constexpr int SB = mf_step_bytes(ACT);
  constexpr int GPB = ACT == QR_Q8_K128 ? 4 : 2;   // groups per activation block
  __shared__ __align__(16) MfStage stage[2];   // double buffer: one barrier per K step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const int64_t t0 = (int64_t)blockIdx.y * MF_TOK;
  const int nsteps = n_in / 128;
  const int64_t x_row_bytes = (int64_t)nsteps * SB;

  // Staging roles: thread tid decodes group tid & 3 of row tid >> 2 (rows
  // of the tile only: with 32 rows, waves 0 and 1), and moves quarter tid & 3
  // (32 code bytes, group tid & 3) of token tid >> 2's step plus one more
  // word of it: Q8_K_128 the scale (quarter 0) or a word of code sums (1,
  // 2); Q8_K64 block 0's scale and sums (0, 1), block 1's (2, 3).
  const int srow = tid >> 2, sq = tid & 3;
  const int64_t grow = r0 + srow < n_out ? r0 + srow : n_out - 1;   // rows past the end: unused
  const uint8_t* wrow = w + grow * w_row_bytes;
  const bool tok_ok = t0 + srow < n_tok;                            // tokens past the end: zeros
  const uint8_t* xrow = x + (tok_ok ? t0 + srow : n_tok - 1) * x_row_bytes;
  // code bytes of group sq, and the extra word (Q8_K_128: quarter 3 repeats 2's)
  const int code_off = ACT == QR_Q8_K128 ? 4 + 32 * sq : 72 * (sq >> 1) + 4 + 32 * (sq & 1);
  const int extra = ACT == QR_Q8_K128 ? (sq == 0 ? 0 : sq == 1 ? 132 : 136)
                                      : (sq == 0 ? 0 : sq == 1 ? 68 : sq == 2 ? 72 : 140);
  RawGroup rg;
  uint32_t av[9];
  // uniform over each wave; always true for 64-row tiles. The load itself is
  // unconditional (rows past the tile load a valid row, not staged), so that
  // the compiler does not wait for it before the step's products.
  const bool wstage = ROWS == MF_ROWS || srow < ROWS;
  auto load_step = [&](int s) {
    rg = load_raw<TYPE>(wrow, 4 * s + sq);
    const uint8_t* blk = xrow + (int64_t)s * SB;
#pragma unroll
    for (int k = 0; k < 8; ++k) av[k] = ld32(blk + code_off + 4 * k);
    av[8] = ld32(blk + extra);
  };
  auto store_step = [&](int s, MfStage& st) {
    if (wstage) {
      const Group G = unpack<TYPE>(rg, 4 * s + sq);
      uint4 c0, c1;
      c0.x = SYM ? signed_levels<TYPE>(G.lo[0]) : G.lo[0];
      c0.y = SYM ? signed_levels<TYPE>(G.lo[1]) : G.lo[1];
      c0.z = SYM ? signed_levels<TYPE>(G.lo[2]) : G.lo[2];
      c0.w = SYM ? signed_levels<TYPE>(G.lo[3]) : G.lo[3];
      c1.x = SYM ? signed_levels<TYPE>(G.hi[0]) : G.hi[0];
      c1.y = SYM ? signed_levels<TYPE>(G.hi[1]) : G.hi[1];
      c1.z = SYM ? signed_levels<TYPE>(G.hi[2]) : G.hi[2];
      c1.w = SYM ? signed_levels<TYPE>(G.hi[3]) : G.hi[3];
      *reinterpret_cast<uint4*>(&st.wq[srow][8 * sq]) = c0;
      *reinterpret_cast<uint4*>(&st.wq[srow][8 * sq + 4]) = c1;
      st.wsa[sq][srow] = G.sa;
      st.wsb[sq][srow] = Q6K ? G.sa1 : (TYPE == QR_Q4_K || TYPE == QR_Q5_K) ? -G.sb : G.sb;
    }
    uint4 a0, a1;
    a0.x = tok_ok ? av[0] : 0u; a0.y = tok_ok ? av[1] : 0u; a0.z = tok_ok ? av[2] : 0u; a0.w = tok_ok ? av[3] : 0u;
    a1.x = tok_ok ? av[4] : 0u; a1.y = tok_ok ? av[5] : 0u; a1.z = tok_ok ? av[6] : 0u; a1.w = tok_ok ? av[7] : 0u;
    *reinterpret_cast<uint4*>(&st.aq[srow][8 * sq]) = a0;
    *reinterpret_cast<uint4*>(&st.aq[srow][8 * sq + 4]) = a1;
    const uint32_t v = tok_ok ? av[8] : 0u;
    const bool is_scale = ACT == QR_Q8_K128 ? sq == 0 : (sq & 1) == 0;
    if (is_scale) {
      st.ad[sq >> 1][srow] = __builtin_bit_cast(float, v);
    } else if (ACT != QR_Q8_K128 || sq < 3) {
      const int g = ACT == QR_Q8_K128 ? 2 * (sq - 1) : sq - 1;   // first of the word's two groups
      st.asum[g][srow] = (float)(int16_t)(v & 0xffffu);
      st.asum[g + 1][srow] = (float)(int16_t)(v >> 16);
    }
  };

  const int wt = (wave & 1) * 32, wr = (wave >> 1) * 16 * RT;   // this wave's tokens and rows in the tile
  const int li = lane & 15, lk = lane >> 4;
  double acc[2][RT][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < RT; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[a][b][v] = 0.0;

  // one step's products from a staged tile
  auto compute = [&](const MfStage& st) {
    // the groups' terms of an activation block, summed in fp32 (at most
    // eight roundings of terms of the block), then scaled and added in double
    float inner[2][RT][4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (gi % GPB == 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < RT; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) inner[a][b][v] = 0.0f;
      }
      long aop[2], bop[RT];
      float sa[RT], sb[RT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        aop[tt] = *reinterpret_cast<const long*>(&st.aq[wt + 16 * tt + li][8 * gi + 2 * lk]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        bop[rt] = *reinterpret_cast<const long*>(&st.wq[wr + 16 * rt + li][8 * gi + 2 * lk]);
        sa[rt] = st.wsa[gi][wr + 16 * rt + li];
        sb[rt] = st.wsb[gi][wr + 16 * rt + li];
      }
      float4 bs[2];
      if (!SYM && !Q6K) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) bs[tt] = *reinterpret_cast<const float4*>(&st.asum[gi][wt + 16 * tt + 4 * lk]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const i32x4 zero = {0, 0, 0, 0};
          if (Q6K) {
            const long blo = lk < 2 ? bop[rt] : 0, bhi = lk < 2 ? 0 : bop[rt];
            const i32x4 dlo = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[tt], blo, zero, 0, 0, 0);
            const i32x4 dhi = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[tt], bhi, zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              inner[tt][rt][v] = __builtin_fmaf(sb[rt], (float)dhi[v], __builtin_fmaf(sa[rt], (float)dlo[v], inner[tt][rt][v]));
          } else {
            const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[tt], bop[rt], zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float t = __builtin_fmaf(sa[rt], (float)d[v], inner[tt][rt][v]);
              if (!SYM) t = __builtin_fmaf(sb[rt], v == 0 ? bs[tt].x : v == 1 ? bs[tt].y : v == 2 ? bs[tt].z : bs[tt].w, t);
              inner[tt][rt][v] = t;
            }
          }
        }
      }
      // the block's activation scale
      if (gi % GPB == GPB - 1) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const float4 d4 = *reinterpret_cast<const float4*>(&st.ad[gi / GPB][wt + 16 * tt + 4 * lk]);
          const double dv[4] = {(double)d4.x, (double)d4.y, (double)d4.z, (double)d4.w};
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[tt][rt][v] = __builtin_fma(dv[v], (double)inner[tt][rt][v], acc[tt][rt][v]);
        }
      }
    }
  };

  // Step s is computed from tile s & 1 while the words of step s + 1 load
  // into registers; they are staged into the other tile afterwards.
  load_step(0);
  store_step(0, stage[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load_step(s + 1);   // in flight during this step's products
    compute(stage[s & 1]);
    if (s + 1 < nsteps) store_step(s + 1, stage[(s + 1) & 1]);
    __syncthreads();   // the next step's tile is staged; this one is free again
  }
  // lanes 16k .. 16k+15 hold consecutive rows of one token: 64-byte runs
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t tok = t0 + wt + 16 * tt + 4 * lk + v;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int64_t row = r0 + wr + 16 * rt + li;
        if (tok < n_tok && row < n_out) y[tok * n_out + row] = (float)acc[tt][rt][v];
      }
    }
}

// Q4_K weights on the matrix cores with the sub-scales folded into the
// integer products. A weight is d sc u - dmin mn (u, sc, mn integers), so one
// activation block's share of an output is
//   d * sum_k sc(k) u_k q_k  -  dmin * sum_k mn(k) q_k,
// two integer dot products over the whole block instead of one per group.
// The first needs sc u as int8: with sc = 8 sh + sl (sh, sl in 0..7) it is
// 8 (sum sh u q) + (sum sl u q), whose operands sh u and sl u are at most
// 105; the second takes mn (at most 63) repeated over the group's 32
// values. So each activation block costs three chains of 16x16x64 products
// (two groups per instruction) accumulated in int32 across its groups
// (exact: each chain's |sum| < 2^21, |8 sum(sh u q) + sum(sl u q)| < 2^24),
// then per output the exact float values of the sums, one product with d
// and one fused multiply-add with dmin: two roundings per block where the
// per-group kernel has up to eight, and fewer vector instructions. The
// weights are staged once as code bytes; each lane forms sl u and sh u from
// them (two multiplies per word), which keeps a workgroup at 42 KB of LDS
// and 168 VGPRs: three workgroups per CU.
template <int ROWS>
struct MfStageK {
  uint32_t aq[MF_TOK][MF_ROW_WORDS];    // activation codes
  uint32_t wu[ROWS][MF_ROW_WORDS];      // weight code bytes u
  uint32_t wsc[ROWS][4];                // per row and group: sc & 7, sc >> 3, mn in bytes 0, 1, 2
  float wd[ROWS], wdm[ROWS];            // d and dmin of the rows' super-block
  double ad[2][MF_TOK];                 // activation scales (of each 64-value block for Q8_K64)
};

// the word that lane k of each group of four lanes holds (DPP quad_perm
// [k, k, k, k])
template <int K>
__device__ __forceinline__ uint32_t quad_word(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, K * 0x55, 0xf, 0xf, false);
}

// An int32 sum that started from the bit pattern of 1.5 * 2^23 (0x4B400000)
// and moved by n, |n| < 2^22, is the float 1.5 * 2^23 + n: the value n is then
// one exact subtraction away, and no conversion instruction is needed.
constexpr int MAGIC_I = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;
__device__ __forceinline__ float magic_value(int biased) { return __builtin_bit_cast(float, biased) - MAGIC_F; }

// codes u (bytes, at most 15) times s (at most 7): no byte carries
__device__ __forceinline__ uint32_t bytes_times(uint32_t u, uint32_t s) { return u * s; }

template <int ACT, int RT>
__global__ __launch_bounds__(MF_THREADS) __attribute__((amdgpu_waves_per_eu(ACT == QR_Q8_K128 ? 3 : 2))) void k_matmul_mfma_q4k(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ x, int64_t n_out, int64_t n_tok, int n_in,
    int64_t w_row_bytes, float* __restrict__ y) {
  constexpr int ROWS = 32 * RT;
  constexpr int SB = mf_step_bytes(ACT);
  constexpr int GPB = ACT == QR_Q8_K128 ? 4 : 2;   // groups per activation block
  __shared__ __align__(16) MfStageK<ROWS> stage[2];   // double buffer: one barrier per K step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const int64_t t0 = (int64_t)blockIdx.y * MF_TOK;
  const int nsteps = n_in / 128;
  const int64_t x_row_bytes = (int64_t)nsteps * SB;

  // staging roles as in k_matmul_mfma: thread tid decodes group tid & 3 of
  // row tid >> 2 and moves quarter tid & 3 of token tid >> 2's step (its 32
  // code bytes, plus the block scale for the quarters that hold one)
  const int srow = tid >> 2, sq = tid & 3;
  const int64_t grow = r0 + srow < n_out ? r0 + srow : n_out - 1;   // rows past the end: unused
  const uint8_t* wrow = w + grow * w_row_bytes;
  const uint8_t* xrow = x + (t0 + srow < n_tok ? t0 + srow : n_tok - 1) * x_row_bytes;
  const int code_off = ACT == QR_Q8_K128 ? 4 + 32 * sq : 72 * (sq >> 1) + 4 + 32 * (sq & 1);
  const bool is_scale = ACT == QR_Q8_K128 ? sq == 0 : (sq & 1) == 0;
  const int scale_off = ACT == QR_Q8_K128 ? 0 : 72 * (sq >> 1);
  uint32_t hdr;   // word sq of the super-block header
  u32x4 codes;    // the group's 16 code bytes
  uint32_t av[9];
  // uniform over each wave; always true for 64-row tiles. The loads are
  // unconditional (rows past the tile load a valid row and are not staged),
  // so that no register they write is touched before the step's products:
  // a conditional load made the compiler wait for it at once.
  const bool wstage = ROWS == MF_ROWS || srow < ROWS;
  auto load_step = [&](int s) {
    // each of a row's four threads loads one word of the super-block header
    // (they are exchanged when staged: one register in flight instead of
    // four, and no four-register tuple for the allocator to split, which
    // made it wait for the load at once), then its group's 16 code bytes
    const int g = 4 * s + sq;
    const uint8_t* sbk = wrow + (int64_t)(g >> 3) * 144;
    hdr = ld32(sbk + 4 * sq);
    codes = *reinterpret_cast<const u32x4*>(sbk + 16 + 16 * (g & 7));
    const uint8_t* blk = xrow + (int64_t)s * SB;
#pragma unroll
    for (int k = 0; k < 8; ++k) av[k] = ld32(blk + code_off + 4 * k);
    av[8] = ld32(blk + scale_off);   // the scale word, used by the quarters that hold one
  };
  auto store_step = [&](int s, MfStageK<ROWS>& st) {
    const uint32_t h0 = quad_word<0>(hdr), h1 = quad_word<1>(hdr), h2 = quad_word<2>(hdr), h3 = quad_word<3>(hdr);
    if (wstage) {
      const int j = (4 * s + sq) & 7;   // the group inside its super-block
      const uint64_t sc6 = (uint64_t)h1 | ((uint64_t)(h2 & 0xffffu) << 32);
      const uint64_t mn6 = (uint64_t)(h2 >> 16) | ((uint64_t)h3 << 16);
      const uint32_t sc = (uint32_t)(sc6 >> (6 * j)) & 63u;
      const uint32_t mn = (uint32_t)(mn6 >> (6 * j)) & 63u;
      const uint32_t c0 = codes[0], c1 = codes[1], c2 = codes[2], c3 = codes[3];
      const uint4 l0 = make_uint4(c0 & 0x0f0f0f0fu, c1 & 0x0f0f0f0fu, c2 & 0x0f0f0f0fu,
                                  c3 & 0x0f0f0f0fu);   // values 0 .. 15 of the group
      const uint4 l1 = make_uint4((c0 >> 4) & 0x0f0f0f0fu, (c1 >> 4) & 0x0f0f0f0fu,
                                  (c2 >> 4) & 0x0f0f0f0fu, (c3 >> 4) & 0x0f0f0f0fu);   // 16 .. 31
      *reinterpret_cast<uint4*>(&st.wu[srow][8 * sq]) = l0;
      *reinterpret_cast<uint4*>(&st.wu[srow][8 * sq + 4]) = l1;
      st.wsc[srow][sq] = (sc & 7u) | ((sc >> 3) << 8) | (mn << 16);
      if (sq == 0) {
        st.wd[srow] = half_bits(h0);
        st.wdm[srow] = half_bits(h0 >> 16);
      }
    }
    // tokens past the end hold the last token's block: each token is its
    // own row of the products, so theirs are never mixed in or stored
    *reinterpret_cast<uint4*>(&st.aq[srow][8 * sq]) = make_uint4(av[0], av[1], av[2], av[3]);
    *reinterpret_cast<uint4*>(&st.aq[srow][8 * sq + 4]) = make_uint4(av[4], av[5], av[6], av[7]);
    if (is_scale) st.ad[sq >> 1][srow] = (double)__builtin_bit_cast(float, av[8]);
  };

  // this wave's tokens and rows in the tile: 64 tokens x 16 rows (64-row
  // tiles) or 32 x 16 (32-row tiles). One 16-row weight operand serves all
  // of the wave's token tiles, so each (row, group) operand is formed by
  // one wave only (64-row tiles) or two.
  constexpr int TW = RT == 2 ? 4 : 2;   // 16-token tiles per wave
  const int wt = RT == 2 ? 0 : (wave & 1) * 32, wr = RT == 2 ? 16 * wave : 16 * (wave >> 1);
  const int li = lane & 15, lk = lane >> 4;
  double acc[TW][4];
#pragma unroll
  for (int a = 0; a < TW; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[a][v] = 0.0;

  // one step's products from a staged tile: per pair of groups (64 values)
  // one 16x16x64 product per chain and token tile; lane l takes the 16
  // values 16 (l / 16) .. +15 of the pair from both operands, so any
  // assignment of the pair's values to operand bytes that is the same for
  // both sides gives the same sum
  auto compute = [&](const MfStageK<ROWS>& st) {
    i32x4 dl[TW], dh[TW], dm[TW];
    const float dw = st.wd[wr + li], dmw = st.wdm[wr + li];
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      if ((2 * gp) % GPB == 0) {
#pragma unroll
        for (int a = 0; a < TW; ++a) {   // each chain's sum is at most 127 * 105 * 128 < 2^21 in magnitude
          dl[a] = i32x4{MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};
          dh[a] = i32x4{MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};
          dm[a] = i32x4{MAGIC_I, MAGIC_I, MAGIC_I, MAGIC_I};
        }
      }
      i32x4 aop[TW];
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
        aop[tt] = *reinterpret_cast<const i32x4*>(&st.aq[wt + 16 * tt + li][16 * gp + 4 * lk]);
      const i32x4 u = *reinterpret_cast<const i32x4*>(&st.wu[wr + li][16 * gp + 4 * lk]);
      // lanes 32..63 hold the pair's second group
      const uint32_t c = st.wsc[wr + li][2 * gp + (lk >> 1)];
      const uint32_t sl = c & 255u, sh = (c >> 8) & 255u;
      const int m = (int)((c >> 16) * 0x01010101u);
      // one weight operand at a time, each used by all token tiles
      const i32x4 blo = i32x4{(int)bytes_times((uint32_t)u[0], sl), (int)bytes_times((uint32_t)u[1], sl),
                              (int)bytes_times((uint32_t)u[2], sl), (int)bytes_times((uint32_t)u[3], sl)};
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) dl[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[tt], blo, dl[tt], 0, 0, 0);
      const i32x4 bhi = i32x4{(int)bytes_times((uint32_t)u[0], sh), (int)bytes_times((uint32_t)u[1], sh),
                              (int)bytes_times((uint32_t)u[2], sh), (int)bytes_times((uint32_t)u[3], sh)};
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) dh[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[tt], bhi, dh[tt], 0, 0, 0);
      const i32x4 bmn = i32x4{m, m, m, m};
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) dm[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[tt], bmn, dm[tt], 0, 0, 0);
      if ((2 * gp + 1) % GPB == GPB - 1) {   // the block's share: d S - dmin O, then the activation scale
        const int blk = (2 * gp + 1) / GPB;
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) {
          const double* dv = &st.ad[blk][wt + 16 * tt + 4 * lk];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // S = 8 sum(sh u q) + sum(sl u q), |S| < 2^24: exact in fp32
            const float S = __builtin_fmaf(8.0f, magic_value(dh[tt][v]), magic_value(dl[tt][v]));
            const float yb = __builtin_fmaf(-dmw, magic_value(dm[tt][v]), dw * S);
            acc[tt][v] = __builtin_fma(dv[v], (double)yb, acc[tt][v]);
          }
        }
      }
      // the next pair's operands are read after this pair's products, which
      // keeps the live registers under the three-workgroup budget
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load_step(0);
  store_step(0, stage[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load_step(s + 1);   // in flight during this step's products
    compute(stage[s & 1]);
    if (s + 1 < nsteps) store_step(s + 1, stage[(s + 1) & 1]);
    __syncthreads();   // the next step's tile is staged; this one is free again
  }
  const int64_t row = r0 + wr + li;
#pragma unroll
  for (int tt = 0; tt < TW; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t tok = t0 + wt + 16 * tt + 4 * lk + v;
      if (tok < n_tok && row < n_out) y[tok * n_out + row] = (float)acc[tt][v];
    }
}

template <int TYPE, int ACT>
int launch_mfma(const uint8_t* w, const uint8_t* x, int64_t n_out, int64_t n_tok, int n_in, int64_t w_row_bytes,
                float* y, hipStream_t s) {
  const int64_t tok_tiles = (n_tok + MF_TOK - 1) / MF_TOK;
  // 64-row tiles unless that leaves fewer than two workgroups per CU
  // (256 CUs): then 32-row tiles, twice as many
  const bool tall = ((n_out + 63) / 64) * tok_tiles >= 512;
  const dim3 grid((uint32_t)(tall ? (n_out + 63) / 64 : (n_out + 31) / 32), (uint32_t)tok_tiles);
  if constexpr (TYPE == QR_Q4_K) {
    if (tall) hipLaunchKernelGGL((k_matmul_mfma_q4k<ACT, 2>), grid, dim3(MF_THREADS), 0, s, w, x, n_out, n_tok, n_in,
                                 w_row_bytes, y);
    else hipLaunchKernelGGL((k_matmul_mfma_q4k<ACT, 1>), grid, dim3(MF_THREADS), 0, s, w, x, n_out, n_tok, n_in,
                            w_row_bytes, y);
    return qr_check_launch("k_matmul_mfma_q4k");
  } else {
    if (tall) hipLaunchKernelGGL((k_matmul_mfma<TYPE, ACT, 2>), grid, dim3(MF_THREADS), 0, s, w, x, n_out, n_tok,
                                 n_in, w_row_bytes, y);
    else hipLaunchKernelGGL((k_matmul_mfma<TYPE, ACT, 1>), grid, dim3(MF_THREADS), 0, s, w, x, n_out, n_tok, n_in,
                            w_row_bytes, y);
    return qr_check_launch("k_matmul_mfma");
  }
}

template <int ACT>
int launch_mfma_type(int t, const uint8_t* w, const uint8_t* x, int64_t n_out, int64_t n_tok, int n_in,
                     int64_t wrb, float* y, hipStream_t s) {
  switch (t) {
    case QR_Q4_0: return launch_mfma<QR_Q4_0, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q4_1: return launch_mfma<QR_Q4_1, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_0: return launch_mfma<QR_Q5_0, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_1: return launch_mfma<QR_Q5_1, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q6_0: return launch_mfma<QR_Q6_0, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q6_K: return launch_mfma<QR_Q6_K, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_K: return launch_mfma<QR_Q5_K, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
    default: return launch_mfma<QR_Q4_K, ACT>(w, x, n_out, n_tok, n_in, wrb, y, s);
  }
}

template <int TYPE, int ACT>
int launch_type(int tt, const uint8_t* w, const uint8_t* x, int64_t n_out, int64_t n_tok, int n_in,
                int64_t w_row_bytes, float* y, hipStream_t s) {
  const int rows = mmq_rows(tt);
  const dim3 grid((uint32_t)((n_out + rows - 1) / rows), (uint32_t)((n_tok + tt - 1) / tt));
  const size_t lds = tt > 1 ? (size_t)mmq_lds_bytes(tt, n_in, ACT) : 0;
  switch (tt) {
    case 8: hipLaunchKernelGGL((k_matmul_q8k<TYPE, ACT, 8>), grid, dim3(MMQ_THREADS), lds, s, w, x, n_out, n_tok, n_in, w_row_bytes, y); break;
    case 4: hipLaunchKernelGGL((k_matmul_q8k<TYPE, ACT, 4>), grid, dim3(MMQ_THREADS), lds, s, w, x, n_out, n_tok, n_in, w_row_bytes, y); break;
    case 2: hipLaunchKernelGGL((k_matmul_q8k<TYPE, ACT, 2>), grid, dim3(MMQ_THREADS), lds, s, w, x, n_out, n_tok, n_in, w_row_bytes, y); break;
    default: hipLaunchKernelGGL((k_matmul_q8k<TYPE, ACT, 1>), grid, dim3(MMQ_THREADS), lds, s, w, x, n_out, n_tok, n_in, w_row_bytes, y); break;
  }
  return qr_check_launch("k_matmul_q8k");
}

template <int ACT>
int launch_act(int t, int tt, const uint8_t* w, const uint8_t* x, int64_t n_out, int64_t n_tok, int n_in,
               int64_t wrb, float* y, hipStream_t s) {
  switch (t) {
    case QR_Q4_0: return launch_type<QR_Q4_0, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q4_1: return launch_type<QR_Q4_1, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_0: return launch_type<QR_Q5_0, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_1: return launch_type<QR_Q5_1, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q6_0: return launch_type<QR_Q6_0, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q6_K: return launch_type<QR_Q6_K, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    case QR_Q5_K: return launch_type<QR_Q5_K, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
    default: return launch_type<QR_Q4_K, ACT>(tt, w, x, n_out, n_tok, n_in, wrb, y, s);
  }
}

}  // namespace

extern "C" {

int qr_matmul_q8k(int t, int act, const void* w, const void* x, int64_t n_out, int64_t n_tok, int64_t n_in,
                  float* y, void* stream) {
  qr_clear_error();
  if (!qr_is_weight_type(t)) return qr_fail(QR_EINVAL_TYPE, "type %d is not a weight-row type", t);
  if (act != QR_Q8_K128 && act != QR_Q8_K64 && act != QR_Q8_K16)
    return qr_fail(QR_EINVAL_TYPE, "activation type %d is not a Q8_K type", act);
  const int64_t wb = (t == QR_Q4_K || t == QR_Q5_K || t == QR_Q6_K) ? 256 : 32;
  const int64_t mult = wb > act_block(act) ? wb : act_block(act);
  if (n_in <= 0 || n_in % mult != 0 || n_in > QR_MATMUL_MAX_IN)
    return qr_fail(QR_EINVAL_SHAPE, "n_in=%lld must be a positive multiple of %lld and at most %d", (long long)n_in,
                   (long long)mult, QR_MATMUL_MAX_IN);
  if (n_out < 0 || n_tok < 0) return qr_fail(QR_EINVAL_SHAPE, "negative n_out or n_tok");
  if (n_out == 0 || n_tok == 0) return QR_OK;
  if (n_out > (int64_t)UINT32_MAX * mmq_rows(1) || n_out > INT64_MAX / n_tok)
    return qr_fail(QR_EOVERFLOW, "n_out or n_tok too large");
  if (!w || !x || !y) return qr_fail(QR_EINVAL_PTR, "w, x and y must be non-NULL");
  if (!qr_aligned(w, 16) || !qr_aligned(x, 16) || !qr_aligned(y, 16))
    return qr_fail(QR_EINVAL_PTR, "device pointers must be 16-byte aligned");
  const int64_t wrb0 = (int64_t)qr_row_bytes(t, n_in);
  if (act != QR_Q8_K16 && n_tok >= MF_MIN_TOK) {   // Q8_K_128 or Q8_K64: the matrix cores
    if ((n_tok + MF_TOK - 1) / MF_TOK > 65535)
      return qr_fail(QR_EOVERFLOW, "n_tok=%lld needs too many token tiles", (long long)n_tok);
    const uint8_t* pw0 = reinterpret_cast<const uint8_t*>(w);
    const uint8_t* px0 = reinterpret_cast<const uint8_t*>(x);
    hipStream_t s0 = reinterpret_cast<hipStream_t>(stream);
    return act == QR_Q8_K128 ? launch_mfma_type<QR_Q8_K128>(t, pw0, px0, n_out, n_tok, (int)n_in, wrb0, y, s0)
                             : launch_mfma_type<QR_Q8_K64>(t, pw0, px0, n_out, n_tok, (int)n_in, wrb0, y, s0);
  }
  // tokens per tile: as many as fit (up to 8) in the activation budget
  int tt = n_tok >= 8 ? 8 : n_tok >= 4 ? 4 : n_tok >= 2 ? 2 : 1;
  while (tt > 1 && mmq_lds_bytes(tt, n_in, act) > MMQ_LDS_BUDGET) tt >>= 1;
  if ((n_tok + tt - 1) / tt > 65535) return qr_fail(QR_EOVERFLOW, "n_tok=%lld needs too many token tiles", (long long)n_tok);
  const int64_t wrb = (int64_t)qr_row_bytes(t, n_in);
  const uint8_t* pw = reinterpret_cast<const uint8_t*>(w);
  const uint8_t* px = reinterpret_cast<const uint8_t*>(x);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (act) {
    case QR_Q8_K64: return launch_act<QR_Q8_K64>(t, tt, pw, px, n_out, n_tok, (int)n_in, wrb, y, s);
    case QR_Q8_K16: return launch_act<QR_Q8_K16>(t, tt, pw, px, n_out, n_tok, (int)n_in, wrb, y, s);
    default: return launch_act<QR_Q8_K128>(t, tt, pw, px, n_out, n_tok, (int)n_in, wrb, y, s);
  }
}

int qr_matmul_q8k128(int t, const void* w, const void* x, int64_t n_out, int64_t n_tok, int64_t n_in, float* y,
                     void* stream) {
  return qr_matmul_q8k(t, QR_Q8_K128, w, x, n_out, n_tok, n_in, y, stream);
}

}  // extern "C"
