// pipe_rates.hip -- instruction rates of the pipes the attention kernel is bound by.
//
// A standalone program (built next to libwattn.so, run by bench.py).  Every workgroup has 8
// waves and two workgroups run per CU, so each SIMD holds 4 waves, as in the attention
// kernel.  Each test kernel repeats one pattern of independent instructions; the program prints
// one JSON line with the time per wave64 instruction per SIMD:
//
//   mfma   v_mfma_f32_16x16x32_bf16, four independent accumulators
//   exp    v_exp_f32, sixteen independent chains
//   fma    v_fma_f32, sixteen independent chains
//   split  half the waves of every SIMD run the mfma pattern, half the fma pattern: equal to
//          the sum of the two when the pipes do not overlap, the larger one when they do
//   inter  one MFMA followed by four exps, four times, in every wave
//
// A softmax-attention step at head dimension 32 needs 128 MFMA flops and one exp per score,
// so the mfma and exp rates give the least time any such kernel spends in the two pipes.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <chrono>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int ITERS = 2048;
constexpr int THREADS = 512;

enum Pattern { P_MFMA = 0, P_EXP = 1, P_FMA = 2, P_INTER = 3 };

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Waves 0-3 of a workgroup run pattern A, waves 4-7 pattern B.  Waves are dealt to the four
// SIMDs of a CU round-robin, so every SIMD receives one wave of each half per workgroup.
template <int A, int B>
__global__ __launch_bounds__(THREADS) void rate_kernel(float* out, float seed) {
  const int pattern = ((threadIdx.x >> 8) & 1) ? B : A;
  const int lane = threadIdx.x & 63;
  const u32x4 a = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f003f00u, 0x3f803f80u};
  const u32x4 b = {0x3f803f80u, 0x3f003f00u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u};
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(lane + i);  // in [0, 1): exp2(-x) stays in (0.5, 1]
  if (pattern == P_MFMA) {
    for (int it = 0; it < ITERS; ++it) {
      c0 = mfma(a, b, c0);
      c1 = mfma(b, a, c1);
      c2 = mfma(a, a, c2);
      c3 = mfma(b, b, c3);
    }
  } else if (pattern == P_EXP) {
    for (int it = 0; it < ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
  } else if (pattern == P_FMA) {
    for (int it = 0; it < ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
    }
  } else {
    for (int it = 0; it < ITERS; ++it) {
      c0 = mfma(a, b, c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      c1 = mfma(b, a, c1);
#pragma unroll
      for (int i = 4; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      c2 = mfma(a, a, c2);
#pragma unroll
      for (int i = 8; i < 12; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      c3 = mfma(b, b, c3);
#pragma unroll
      for (int i = 12; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
  }
  float s = c0[0] + c1[1] + c2[2] + c3[3];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

struct Ctx {
  float* buf;
  int blocks;
  hipEvent_t e0, e1;
};

template <int A, int B>
bool time_kernel(Ctx& C, int reps, float* best_ms) {
  float best = 1e30f;
  for (int r = 0; r < reps; ++r) {
    if (hipEventRecord(C.e0, nullptr) != hipSuccess) return false;
    hipLaunchKernelGGL((rate_kernel<A, B>), dim3(C.blocks), dim3(THREADS), 0, nullptr, C.buf, 1.0f / 128.0f);
    if (hipGetLastError() != hipSuccess) return false;
    if (hipEventRecord(C.e1, nullptr) != hipSuccess) return false;
    if (hipEventSynchronize(C.e1) != hipSuccess) return false;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, C.e0, C.e1) != hipSuccess) return false;
    if (ms < best) best = ms;
  }
  *best_ms = best;
  return true;
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) {
    fprintf(stderr, "pipe_rates: no HIP device\n");
    return 1;
  }
  Ctx C;
  C.blocks = 2 * prop.multiProcessorCount;  // 16 waves per CU = 4 per SIMD
  const int simds = 4 * prop.multiProcessorCount;
  if (hipMalloc(&C.buf, (size_t)C.blocks * THREADS * sizeof(float)) != hipSuccess) return 1;
  if (hipEventCreate(&C.e0) != hipSuccess || hipEventCreate(&C.e1) != hipSuccess) return 1;

  // bring the clocks up: half a second of back-to-back launches
  const auto t0 = std::chrono::steady_clock::now();
  while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < 0.5) {
    for (int i = 0; i < 20; ++i)
      hipLaunchKernelGGL((rate_kernel<P_MFMA, P_EXP>), dim3(C.blocks), dim3(THREADS), 0, nullptr, C.buf, 0.01f);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
  }

  float t_mfma, t_exp, t_fma, t_split, t_inter;
  const int reps = 5;
  if (!time_kernel<P_MFMA, P_MFMA>(C, reps, &t_mfma) || !time_kernel<P_EXP, P_EXP>(C, reps, &t_exp) ||
      !time_kernel<P_FMA, P_FMA>(C, reps, &t_fma) || !time_kernel<P_MFMA, P_FMA>(C, reps, &t_split) ||
      !time_kernel<P_INTER, P_INTER>(C, reps, &t_inter)) {
    fprintf(stderr, "pipe_rates: a HIP call failed\n");
    return 1;
  }
  // wave64 instructions of one pattern per SIMD: 4 waves x ITERS iterations x (4 or 16)
  const double waves_per_simd = (double)C.blocks * (THREADS / 64) / simds;
  const double it_per_simd = waves_per_simd * ITERS;
  const double ns = 1e6;  // ms -> ns
  printf("{\"simds\": %d, \"waves_per_simd\": %.0f, \"ns_per_instruction\": {\"mfma_f32_16x16x32_bf16\": %.4f, "
         "\"exp_f32\": %.4f, \"fma_f32\": %.4f}, \"split_mfma_fma_ns_per_iteration\": %.4f, "
         "\"serial_mfma_fma_ns_per_iteration\": %.4f, \"interleaved_4mfma_16exp_ns\": %.4f, "
         "\"serial_4mfma_16exp_ns\": %.4f}\n",
         simds, waves_per_simd, t_mfma * ns / (it_per_simd * 4), t_exp * ns / (it_per_simd * 16),
         t_fma * ns / (it_per_simd * 16), t_split * ns / it_per_simd,
         0.5 * (t_mfma + t_fma) * ns / it_per_simd, t_inter * ns / it_per_simd, (t_mfma + t_exp) * ns / it_per_simd);
  return 0;
}
