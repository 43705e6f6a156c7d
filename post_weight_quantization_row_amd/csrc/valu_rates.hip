// valu_rates.hip -- measurement only (libqrow_probe.so): issue rates of the
// vector-ALU instruction classes the row quantizer is made of, on the GPU
// the benchmark runs on. Not part of the quantization path.
//
// Each kernel runs a fixed, unrolled sequence of one instruction class on
// register operands only (no memory traffic inside the timed loop): eight
// independent dependency chains per lane, or one chain, at a chosen number
// of waves per SIMD. The host times the launch with HIP events and reports
// SIMD cycles per wave64 instruction at the nominal 2.4 GHz clock. These
// rates calibrate the VALU figures reported beside the HBM roofline: gfx950
// issues two VALU instructions per cycle per SIMD for some classes (the
// SQ_ACTIVE_INST_VALU2 counter counts those cycles), so a model that charges
// every wave64 instruction four cycles overstates the VALU time.

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

enum {
  K_FMA_F32 = 0,     // v_fma_f32, 8 chains
  K_ADD_F32,         // v_add_f32, 8 chains
  K_XOR_B32,         // v_xor_b32, 8 chains
  K_RNDNE_F32,       // v_rndne_f32, 8 chains
  K_MED3_F32,        // v_med3_f32, 8 chains
  K_CMP_CNDMASK,     // v_cmp_lt_f32 + v_cndmask_b32, 8 chains
  K_FMA_RNDNE,       // v_fma_f32 and v_rndne_f32 interleaved, 8 chains
  K_FMA_F64,         // v_fma_f64, 4 chains
  K_SQRT_F32,        // v_sqrt_f32, 8 chains
  K_FMA_F32_CHAIN,   // v_fma_f32, one chain
  K_COUNT
};

// wave64 instructions per lane per iteration of each kernel
__host__ __device__ constexpr int instr_per_iter(int k) {
  return k == K_CMP_CNDMASK || k == K_FMA_RNDNE ? 128 : 64;
}

template <int K>
__global__ __launch_bounds__(256) void k_rates(const float* __restrict__ in, float* __restrict__ sink, int iters) {
  float a[8];
  uint32_t u[8];
  double d[4];
  const float b = in[0], c = in[1];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (float)threadIdx.x * 1e-3f + (float)i;
    u[i] = threadIdx.x + i;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = a[i];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (K == K_FMA_F32) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (K == K_ADD_F32) asm volatile("v_add_f32 %0, %1, %0" : "+v"(a[i]) : "v"(b));
        if constexpr (K == K_XOR_B32) asm volatile("v_xor_b32 %0, %1, %0" : "+v"(u[i]) : "v"(u[(i + 1) & 7]));
        if constexpr (K == K_RNDNE_F32) asm volatile("v_rndne_f32 %0, %0" : "+v"(a[i]));
        if constexpr (K == K_MED3_F32) asm volatile("v_med3_f32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        if constexpr (K == K_CMP_CNDMASK)
          asm volatile("v_cmp_lt_f32 vcc, %0, %1\n\tv_cndmask_b32 %0, %0, %1, vcc" : "+v"(a[i]) : "v"(b) : "vcc");
        if constexpr (K == K_FMA_RNDNE) {
          asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(a[i]) : "v"(b), "v"(c));
          asm volatile("v_rndne_f32 %0, %1" : "=v"(a[(i + 4) & 7]) : "v"(a[(i + 3) & 7]));
        }
        if constexpr (K == K_FMA_F64)
          asm volatile("v_fma_f64 %0, %1, %2, %0" : "+v"(d[i & 3]) : "v"((double)b), "v"((double)c));
        if constexpr (K == K_SQRT_F32) asm volatile("v_sqrt_f32 %0, %0" : "+v"(a[i]));
        if constexpr (K == K_FMA_F32_CHAIN) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(a[0]) : "v"(b), "v"(c));
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] + (float)u[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)d[i];
  if (s == 1234.5f) sink[blockIdx.x] = s;   // keeps the chains alive; practically never stored
}

template <int K>
int time_one(const float* in, float* sink, int waves_per_simd, int n_simds, float* cycles) {
  const int iters = 256;
  const int blocks = n_simds * waves_per_simd / 4;   // four waves per 256-thread block
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1;
  hipLaunchKernelGGL(k_rates<K>, dim3(blocks), dim3(256), 0, 0, in, sink, 4);   // warm-up
  hipEventRecord(e0, 0);
  hipLaunchKernelGGL(k_rates<K>, dim3(blocks), dim3(256), 0, 0, in, sink, iters);
  hipEventRecord(e1, 0);
  float ms = 0.0f;
  const bool ok = hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
                  hipGetLastError() == hipSuccess;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (!ok) return -1;
  const double instr = (double)blocks * 4.0 * iters * instr_per_iter(K);   // wave64 instructions
  *cycles = (float)(ms * 1e-3 * 2.4e9 * n_simds / instr);
  return 0;
}

}  // namespace

extern "C" {

// Number of instruction classes qrp_valu_rates measures.
int qrp_valu_classes(void) { return K_COUNT; }

// SIMD cycles per wave64 instruction (at 2.4 GHz) of every class, at
// `waves_per_simd` waves per SIMD (1..8) on `n_simds` SIMDs (4 per compute
// unit). `in` is a device buffer of two floats (operands), `sink` a device
// buffer of n_simds * waves_per_simd / 4 floats that is practically never
// written. Runs on the null stream; returns 0, or -1 on a HIP error.
int qrp_valu_rates(const float* in, float* sink, int waves_per_simd, int n_simds, float* cycles_out) {
  if (waves_per_simd < 1 || waves_per_simd > 8 || n_simds < 4 || n_simds % 4) return -1;
  int rc = 0;
  rc |= time_one<K_FMA_F32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_FMA_F32]);
  rc |= time_one<K_ADD_F32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_ADD_F32]);
  rc |= time_one<K_XOR_B32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_XOR_B32]);
  rc |= time_one<K_RNDNE_F32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_RNDNE_F32]);
  rc |= time_one<K_MED3_F32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_MED3_F32]);
  rc |= time_one<K_CMP_CNDMASK>(in, sink, waves_per_simd, n_simds, &cycles_out[K_CMP_CNDMASK]);
  rc |= time_one<K_FMA_RNDNE>(in, sink, waves_per_simd, n_simds, &cycles_out[K_FMA_RNDNE]);
  rc |= time_one<K_FMA_F64>(in, sink, waves_per_simd, n_simds, &cycles_out[K_FMA_F64]);
  rc |= time_one<K_SQRT_F32>(in, sink, waves_per_simd, n_simds, &cycles_out[K_SQRT_F32]);
  rc |= time_one<K_FMA_F32_CHAIN>(in, sink, waves_per_simd, n_simds, &cycles_out[K_FMA_F32_CHAIN]);
  return rc ? -1 : 0;
}

}  // extern "C"
