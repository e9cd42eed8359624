// access_rates -- HBM rate of the small-window attention's memory access pattern, with the
// attention taken out (a measurement program built beside libwattn.so; bench.py does not use it).
//
// q, k, v: [16][128][128][3][32] bf16 and out [16][128][128][3][32] fp32, cut into 8 x 8 windows:
// the shape of the 16 x 128 x 128, 3-head, M = 8 workload.  Three sets of the four tensors
// (756 MB) rotate from launch to launch, so that no launch finds its data in the 256 MB
// last-level cache.  Every kernel reads q, k, v once and writes out = q + k + v once (252 MB).
//   per_head     : one 128-thread workgroup per (window, head), as the attention kernel at
//                  M = 8 is laid out: each token contributes a 64-byte piece at a 192-byte
//                  stride, and the three heads of a token are read by three workgroups;
//   whole_tokens : one 384-thread workgroup per window: each token's 192 bytes are read as one
//                  contiguous run by consecutive threads;
//   per_head_xcd : per_head with the workgroups dealt to the XCDs as the attention kernel deals
//                  its tasks: runs of 16 consecutive (window, head) tasks to one XCD, so the
//                  three heads of a token meet in one L2;
//   per_head_x2  : per_head with two windows of the same head per workgroup: twice the loads in
//                  flight per thread;
//   copy         : a plain element-wise copy, 50 MB read and 50 MB written (grid-stride loop).
// Prints one line per kernel: average microseconds per launch over 100 launches after 300 of
// warm-up, and the rate against 8 TB/s.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int B = 16, G = 128, H = 3, D = 32, M = 8, NWS = G / M;

__device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// out[0..7] = q + k + v for eight bf16 channels
__device__ __forceinline__ void emit(float* o, u32x4 a, u32x4 b, u32x4 c) {
  const float4 r0 = make_float4(lo(a[0]) + lo(b[0]) + lo(c[0]), hi(a[0]) + hi(b[0]) + hi(c[0]),
                                lo(a[1]) + lo(b[1]) + lo(c[1]), hi(a[1]) + hi(b[1]) + hi(c[1]));
  const float4 r1 = make_float4(lo(a[2]) + lo(b[2]) + lo(c[2]), hi(a[2]) + hi(b[2]) + hi(c[2]),
                                lo(a[3]) + lo(b[3]) + lo(c[3]), hi(a[3]) + hi(b[3]) + hi(c[3]));
  reinterpret_cast<float4*>(o)[0] = r0;
  reinterpret_cast<float4*>(o)[1] = r1;
}

// element offset of token i (0..63, row-major in the window) of window w, plus `inner`
__device__ __forceinline__ int64_t token_offset(int w, int i, int inner) {
  const int b = w / (NWS * NWS), wy = (w / NWS) % NWS, wx = w % NWS;
  const int y = wy * M + i / M, x = wx * M + i % M;
  return ((int64_t)(b * G + y) * G + x) * (H * D) + inner;
}

template <bool XCD>
__global__ __launch_bounds__(128) void gather_per_head(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, float* __restrict__ out) {
  // workgroups are dealt to the 8 XCDs round-robin; with XCD, slot s of XCD x takes task
  // (s / 16 * 8 + x) * 16 + s % 16 (the grid is a multiple of 128)
  const int bid = blockIdx.x;
  const int task = XCD ? (((bid >> 3) / 16 * 8 + (bid & 7)) * 16 + (bid >> 3) % 16) : bid;
  const int w = task / H, h = task % H, t = threadIdx.x;
  u32x4 a[2], b[2], c[2];
  int64_t off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {  // thread t: 16-byte chunk t % 4 of tokens t / 4 and t / 4 + 32
    off[r] = token_offset(w, (t >> 2) + 32 * r, h * D + (t & 3) * 8);
    a[r] = *reinterpret_cast<const u32x4*>(q + off[r]);
    b[r] = *reinterpret_cast<const u32x4*>(k + off[r]);
    c[r] = *reinterpret_cast<const u32x4*>(v + off[r]);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) emit(out + off[r], a[r], b[r], c[r]);
}

__global__ __launch_bounds__(384) void gather_whole_tokens(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, float* __restrict__ out) {
  const int w = blockIdx.x, t = threadIdx.x;
  u32x4 a[2], b[2], c[2];
  int64_t off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {  // thread t: 16-byte chunk t % 12 of tokens t / 12 and t / 12 + 32
    off[r] = token_offset(w, t / 12 + 32 * r, (t % 12) * 8);
    a[r] = *reinterpret_cast<const u32x4*>(q + off[r]);
    b[r] = *reinterpret_cast<const u32x4*>(k + off[r]);
    c[r] = *reinterpret_cast<const u32x4*>(v + off[r]);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) emit(out + off[r], a[r], b[r], c[r]);
}

__global__ __launch_bounds__(128) void gather_per_head_x2(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, float* __restrict__ out) {
  const int w0 = (blockIdx.x / H) * 2, h = blockIdx.x % H, t = threadIdx.x;
  u32x4 a[4], b[4], c[4];
  int64_t off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {  // windows w0 and w0 + 1, each as in gather_per_head
    off[r] = token_offset(w0 + (r >> 1), (t >> 2) + 32 * (r & 1), h * D + (t & 3) * 8);
    a[r] = *reinterpret_cast<const u32x4*>(q + off[r]);
    b[r] = *reinterpret_cast<const u32x4*>(k + off[r]);
    c[r] = *reinterpret_cast<const u32x4*>(v + off[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) emit(out + off[r], a[r], b[r], c[r]);
}

__global__ __launch_bounds__(256) void copy_f4(const float4* __restrict__ s, float4* __restrict__ d, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}

}  // namespace

#define CHECK(x)                                                                   \
  do {                                                                             \
    const hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

int main() {
  const int64_t n = (int64_t)B * G * G * H * D;  // elements per tensor
  uint16_t *qs[3], *ks[3], *vs[3];
  float* os[3];
  for (int s = 0; s < 3; ++s) {
    CHECK(hipMalloc(&qs[s], n * 2));
    CHECK(hipMalloc(&ks[s], n * 2));
    CHECK(hipMalloc(&vs[s], n * 2));
    CHECK(hipMalloc(&os[s], n * 4));
    CHECK(hipMemset(qs[s], 0, n * 2));
    CHECK(hipMemset(ks[s], 0, n * 2));
    CHECK(hipMemset(vs[s], 0, n * 2));
    CHECK(hipMemset(os[s], 0, n * 4));
  }
  const int nwin = B * NWS * NWS;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const char* names[5] = {"per_head", "whole_tokens", "per_head_x2", "copy", "per_head_xcd"};
  int it = 0;
  for (int which = 0; which < 5; ++which) {
    auto launch = [&]() {
      const int s = (it++) % 3;
      if (which == 0)
        hipLaunchKernelGGL(gather_per_head<false>, dim3(nwin * H), dim3(128), 0, 0, qs[s], ks[s], vs[s], os[s]);
      else if (which == 4)  // nwin * H = 12288 is a multiple of 128
        hipLaunchKernelGGL(gather_per_head<true>, dim3(nwin * H), dim3(128), 0, 0, qs[s], ks[s], vs[s], os[s]);
      else if (which == 1)
        hipLaunchKernelGGL(gather_whole_tokens, dim3(nwin), dim3(384), 0, 0, qs[s], ks[s], vs[s], os[s]);
      else if (which == 2)  // nwin is even
        hipLaunchKernelGGL(gather_per_head_x2, dim3(nwin / 2 * H), dim3(128), 0, 0, qs[s], ks[s], vs[s], os[s]);
      else  // 50 MB of set s's out copied into its q buffer: 100 MB of traffic
        hipLaunchKernelGGL(copy_f4, dim3(4096), dim3(256), 0, 0, reinterpret_cast<const float4*>(os[s]),
                           reinterpret_cast<float4*>(qs[s]), n * 2 / 16);
    };
    for (int i = 0; i < 300; ++i) launch();
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int i = 0; i < 100; ++i) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double us = ms * 1e3 / 100;
    const double bytes = which == 3 ? 2.0 * n * 2 : 3.0 * n * 2 + 4.0 * n;
    printf("%-13s %8.1f us  %6.0f GB/s  %5.1f%% of 8 TB/s\n", names[which], us, bytes / us * 1e-3,
           bytes / us * 1e-3 / 80.0);
  }
  return 0;
}
