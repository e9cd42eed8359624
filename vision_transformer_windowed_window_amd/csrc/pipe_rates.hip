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
//   expfma sixteen exps and sixteen independent FMAs interleaved in every wave: equal to the
//          sum of the exp and fma patterns when the two do not overlap
//   step   the instruction mix of one 32-key step of the attention kernel per wave (two
//          16-query blocks at d = 32): four fp16 score MFMAs, 16 exps, 8 bf16 packs, the bit
//          test of the lazy rescale, four bf16 value MFMAs and two row-sum MFMAs, with its
//          LDS fragment reads; the least time per step of the attention kernel's steady state
//   pstep  the same step software-pipelined: the score MFMAs of step t+1 are issued before the
//          exponentials of step t (two score sets live, 16 more registers)
//   clock  the shader clock while every SIMD runs MFMAs: the shader-cycle counter (s_memtime)
//          against the 100 MHz real-time counter (s_memrealtime), read by every workgroup
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int ITERS = 2048;
constexpr int THREADS = 512;

enum Pattern { P_MFMA = 0, P_EXP = 1, P_FMA = 2, P_INTER = 3, P_EXPFMA = 4 };

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
  float x[16], y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = seed * (float)(lane + i);  // in [0, 1): exp2(-x) stays in (0.5, 1]
    y[i] = seed * (float)(lane + 2 * i);
  }
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
  } else if (pattern == P_EXPFMA) {
    for (int it = 0; it < ITERS; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
        y[i] = fmaf(y[i], 0.999f, 0.001f);
      }
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
  for (int i = 0; i < 16; ++i) s += x[i] + y[i];
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

// Every workgroup runs the MFMA pattern for CLOCK_ITERS iterations and records both counters
// before and after (thread 0 only); the host averages cycles / real time over the workgroups.
constexpr int CLOCK_ITERS = 16384;
__global__ __launch_bounds__(THREADS) void clock_kernel(unsigned long long* stamps, float* out) {
  const int lane = threadIdx.x & 63;
  const u32x4 a = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f003f00u, 0x3f803f80u};
  const u32x4 b = {0x3f803f80u, 0x3f003f00u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u};
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < CLOCK_ITERS; ++it) {
    c0 = mfma(a, b, c0);
    c1 = mfma(b, a, c1);
    c2 = mfma(a, a, c2);
    c3 = mfma(b, b, c3);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    stamps[4 * blockIdx.x + 0] = t1 - t0;
    stamps[4 * blockIdx.x + 1] = r1 - r0;
  }
}

// One attention step per iteration (see the header); the probabilities stay below 2^-16, so
// the rescale branch is never taken, as in the kernel's steady state.
constexpr int STEP_ITERS = 512;
template <bool PIPE>
__global__ __launch_bounds__(THREADS) void step_kernel(float* out, float seed) {
  __shared__ __align__(16) uint16_t sK[2][128 * 32];
  __shared__ __align__(16) uint16_t sV[2][128 * 32];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
  for (int i = tid; i < 2 * 128 * 32; i += THREADS) {
    (&sK[0][0])[i] = (uint16_t)(0x2c00 + (i & 0x3ff));  // fp16 around 0.06
    (&sV[0][0])[i] = (uint16_t)(0x3c00 + (i & 0x7f));   // bf16 around 0.008
  }
  __syncthreads();
  const u32x4 Q[2] = {{0x2c002c00u + lane, 0x2c002c00u, 0x2c002c00u, 0x2c002c00u},
                      {0x2c002c00u, 0x2c002c00u + lane, 0x2c002c00u, 0x2c002c00u}};
  const u32x4 ONES4 = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const float r = seed + 16.f;
  const f32x4 Cn = {-r, -r, -r, -r};
  f32x4 O[2][2] = {}, L[2] = {};
  int flag = 0;
  // K fragments of step t (rows kb .. kb + 31 of buffer t % 2, kb = 32 (t % 4): inside the tile)
  auto kfrags = [&](int t, u32x4 (&Kf)[2]) {
    const int buf = t & 1, kb = (t & 3) * 32;
#pragma unroll
    for (int b = 0; b < 2; ++b)
      Kf[b] = *reinterpret_cast<const u32x4*>(&sK[buf][(kb + 8 * (c >> 2) + (c & 3) + 4 * b) * 32 + g * 8]);
  };
  auto scores = [&](const u32x4 (&Kf)[2], f32x4 (&S)[2][2]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        S[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Kf[b]),
                                                          __builtin_bit_cast(f16x8, Q[a]), Cn, 0, 0, 0);
  };
  f32x4 Snext[2][2];
  if (PIPE) {
    u32x4 K0[2];
    kfrags(0, K0);
    scores(K0, Snext);
  }
#pragma unroll(PIPE ? 2 : 1)
  for (int t = 0; t < STEP_ITERS; ++t) {
    const int buf = t & 1, kb = (t & 3) * 32;
    u32x4 Kf[2], Vf[2];
    f32x4 S[2][2];
    if (PIPE) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) S[a][b] = Snext[a][b];
      kfrags(t + 1, Kf);
      scores(Kf, Snext);  // step t + 1, issued before the exponentials of step t
    } else {
      kfrags(t, Kf);
      scores(Kf, S);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      u32x2 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint16_t* p = &sV[buf][(kb + 8 * g + (c >> 2) + 4 * hh) * 32 + 16 * db + 4 * (c & 1)];
        h[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                              (lds_i16x4*)(__attribute__((address_space(3))) void*)(p)));
      }
      Vf[db] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
    }
    uint32_t P[2][4], bits = 0u;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 f = {__builtin_amdgcn_exp2f(S[a][i >> 1][2 * (i & 1)]),
                         __builtin_amdgcn_exp2f(S[a][i >> 1][2 * (i & 1) + 1])};
        P[a][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
        bits |= P[a][i];
      }
    if (__any((bits & 0x40004000u) != 0u)) {  // never taken here
      ++flag;
      O[0][0] *= 0.5f;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const u32x4 Pa = {P[a][0], P[a][1], P[a][2], P[a][3]};
#pragma unroll
      for (int db = 0; db < 2; ++db) O[db][a] = mfma(Vf[db], Pa, O[db][a]);
      L[a] = mfma(ONES4, Pa, L[a]);
    }
  }
  out[(size_t)blockIdx.x * THREADS + tid] = O[0][0][0] + O[1][1][3] + L[0][1] + L[1][2] + (float)flag;
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
  float t_expfma;
  if (!time_kernel<P_EXPFMA, P_EXPFMA>(C, reps, &t_expfma)) {
    fprintf(stderr, "pipe_rates: a HIP call failed\n");
    return 1;
  }
  // attention step, plain and software-pipelined
  float t_step = 1e30f, t_pstep = 1e30f;
  for (int r = 0; r < reps; ++r) {
    for (int pipe = 0; pipe < 2; ++pipe) {
      if (hipEventRecord(C.e0, nullptr) != hipSuccess) return 1;
      if (pipe)
        hipLaunchKernelGGL(step_kernel<true>, dim3(C.blocks), dim3(THREADS), 0, nullptr, C.buf, 0.5f);
      else
        hipLaunchKernelGGL(step_kernel<false>, dim3(C.blocks), dim3(THREADS), 0, nullptr, C.buf, 0.5f);
      if (hipEventRecord(C.e1, nullptr) != hipSuccess || hipEventSynchronize(C.e1) != hipSuccess) return 1;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, C.e0, C.e1) != hipSuccess) return 1;
      float& best = pipe ? t_pstep : t_step;
      if (ms < best) best = ms;
    }
  }

  // shader clock under MFMA load (cycles of s_memtime per 10 ns tick of s_memrealtime)
  unsigned long long* stamps = nullptr;
  if (hipMalloc(&stamps, (size_t)C.blocks * 4 * sizeof(unsigned long long)) != hipSuccess) return 1;
  hipLaunchKernelGGL(clock_kernel, dim3(C.blocks), dim3(THREADS), 0, nullptr, stamps, C.buf);
  if (hipDeviceSynchronize() != hipSuccess) return 1;
  unsigned long long* hs = new unsigned long long[(size_t)C.blocks * 4];
  if (hipMemcpy(hs, stamps, (size_t)C.blocks * 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return 1;
  double cyc = 0.0, ticks = 0.0;
  for (int i = 0; i < C.blocks; ++i) {
    cyc += (double)hs[4 * i];
    ticks += (double)hs[4 * i + 1];
  }
  const double sclk_ghz = ticks > 0.0 ? cyc / ticks * 0.1 : 0.0;  // real-time counter: 100 MHz
  delete[] hs;

  // wave64 instructions of one pattern per SIMD: 4 waves x ITERS iterations x (4 or 16)
  const double waves_per_simd = (double)C.blocks * (THREADS / 64) / simds;
  const double it_per_simd = waves_per_simd * ITERS;
  const double ns = 1e6;  // ms -> ns
  printf("{\"simds\": %d, \"shader_clock_ghz_mfma_load\": %.4f, \"waves_per_simd\": %.0f, \"ns_per_instruction\": {\"mfma_f32_16x16x32_bf16\": %.4f, "
         "\"exp_f32\": %.4f, \"fma_f32\": %.4f}, \"split_mfma_fma_ns_per_iteration\": %.4f, "
         "\"serial_mfma_fma_ns_per_iteration\": %.4f, \"interleaved_4mfma_16exp_ns\": %.4f, "
         "\"serial_4mfma_16exp_ns\": %.4f, \"expfma_same_wave_ns_per_iteration\": %.4f, "
         "\"serial_exp_fma_ns_per_iteration\": %.4f, \"softmax_step_ns\": %.3f, "
         "\"softmax_step_pipelined_ns\": %.3f}\n",
         simds, sclk_ghz, waves_per_simd, t_mfma * ns / (it_per_simd * 4), t_exp * ns / (it_per_simd * 16),
         t_fma * ns / (it_per_simd * 16), t_split * ns / it_per_simd,
         0.5 * (t_mfma + t_fma) * ns / it_per_simd, t_inter * ns / it_per_simd, (t_mfma + t_exp) * ns / it_per_simd,
         t_expfma * ns / it_per_simd, (t_exp + t_fma) * ns / it_per_simd,
         t_step * ns / (waves_per_simd * STEP_ITERS), t_pstep * ns / (waves_per_simd * STEP_ITERS));
  return 0;
}
