// wattn_model.hip -- the model steps around the window attention (gfx950): linear layers with
// fused epilogues, layer norm (optionally over gathered 2 x 2 neighbours), the overlapping stem
// convolution and the token mean of the classifier.
//
// FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with Memory
// Efficient Attention -- "How it works": Swin's hierarchy is kept; the patch embedding becomes
// an overlapping convolution with kernel 2p - 1, stride p and padding p - 1.
//
// Layouts: activations are token-major bf16 [tokens][channels] (the attention's
// [B][Hg][Wg][H][d] with C = H * d); weights of linear layers bf16 [out][in]; biases, norm gains
// and norm biases fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wattn_plan.h"

namespace {

#include "wattn_device.h"

// ---------------------------------------------------------------------------------------
// y = act(x W^T + b) (+ res).  One wave per workgroup computes 32 tokens x 64 outputs as
// y^T = W x^T: 16x16x32 bf16 MFMA with A = 16 rows of W (8 consecutive inputs per lane, read
// straight from global memory: W is small and stays in the caches) and B = 16 tokens of x.  A
// lane's accumulator holds four consecutive outputs of one token, stored as 8 bytes.  The
// operands of the next k step are loaded while the current one multiplies.  Output column n
// goes to part n / split at offset part * part_stride + m * split + n % split, which writes
// q, k and v of a qkv projection as three separate [M][C] tensors.
// ---------------------------------------------------------------------------------------

enum { ACT_NONE = 0, ACT_GELU = 1 };

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

template <int ACT, bool RES, bool OUTF32>
__global__ __launch_bounds__(64) void wattn_linear_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          const uint16_t* res, void* y, const LinearPlan P) {
  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 64;
  // rows this lane reads: tokens m0 + 16 mb + c, outputs n0 + 16 nb + c
  const uint16_t* xr[2];
  const uint16_t* wr[4];
  bool xv[2], wv[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 16 * mb + c;
    xv[mb] = m < P.M;
    xr[mb] = x + (int64_t)(xv[mb] ? m : 0) * P.K + 8 * g;
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + c;
    wv[nb] = n < P.N;
    wr[nb] = W + (int64_t)(wv[nb] ? n : 0) * P.K + 8 * g;
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto load = [&](int k0, u32x4 (&xa)[2], u32x4 (&wa)[4]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) xa[mb] = xv[mb] ? *reinterpret_cast<const u32x4*>(xr[mb] + k0) : zero4;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) wa[nb] = wv[nb] ? *reinterpret_cast<const u32x4*>(wr[nb] + k0) : zero4;
  };
  f32x4 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 xa[2], wa[4], xb[2], wb[4];
  load(0, xa, wa);
  for (int k0 = 0; k0 < P.K; k0 += 64) {
    const bool more = k0 + 32 < P.K;
    if (more) load(k0 + 32, xb, wb);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma16_bf16(wa[nb], xa[mb], acc[nb][mb]);
    if (!more) break;
    if (k0 + 64 < P.K) load(k0 + 64, xa, wa);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma16_bf16(wb[nb], xb[mb], acc[nb][mb]);
  }
  // epilogue: lane (c, g) holds outputs n0 + 16 nb + 4 g + e of token m0 + 16 mb + c
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 16 * mb + c;
    if (m >= P.M) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + 16 * nb + 4 * g;
      if (n >= P.N) continue;
      const int part = n / P.split, nn = n - part * P.split;
      const int64_t off = (int64_t)part * P.part_stride + (int64_t)m * P.split + nn;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = acc[nb][mb][e] + (bias != nullptr ? bias[n + e] : 0.f);
        if (ACT == ACT_GELU) t = gelu_erf(t);
        r[e] = t;
      }
      if (RES) {
        const u32x2 rv = *reinterpret_cast<const u32x2*>(res + off);
        r[0] += bf_lo(rv[0]);
        r[1] += bf_hi(rv[0]);
        r[2] += bf_lo(rv[1]);
        r[3] += bf_hi(rv[1]);
      }
      if (OUTF32) {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = make_float4(r[0], r[1], r[2], r[3]);
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + off) =
            u32x2{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Layer norm over the channels of each token, 16 lanes per token (4 tokens per wave): fp32
// sums of x and x^2 over the 16-byte chunks of the row, a reduction over the lane group, then a
// second pass over the (cached) row that normalises and writes bf16.  GATHER: the row of output
// token (b, i, j) is the concatenation of input tokens (2i, 2j), (2i+1, 2j), (2i, 2j+1),
// (2i+1, 2j+1) of a [B][Hg][Wg][C] map (patch merging).
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

template <bool GATHER>
__global__ __launch_bounds__(256) void wattn_layernorm_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ gamma,
                                                              const float* __restrict__ beta,
                                                              uint16_t* __restrict__ y, const NormPlan P) {
  const int tid = threadIdx.x, l16 = tid & 15;
  const int64_t t = (int64_t)blockIdx.x * 16 + (tid >> 4);  // output token
  if (t >= P.T) return;
  const int Ct = GATHER ? 4 * P.C : P.C;  // channels of the normalised row
  const int nch = Ct / 8;
  // address of chunk j (8 channels) of the row
  int64_t src[4];
  if (GATHER) {
    const int Wo = P.Wg / 2, Ho = P.Hg / 2;
    const int64_t b = t / ((int64_t)Ho * Wo);
    const int rem = (int)(t - b * Ho * Wo);
    const int i = rem / Wo, jx = rem - i * Wo;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      src[qd] = ((b * P.Hg + 2 * i + (qd & 1)) * P.Wg + 2 * jx + (qd >> 1)) * P.C;
  } else {
    src[0] = t * P.C;
  }
  auto chunk_ptr = [&](int j) -> const uint16_t* {
    if (!GATHER) return x + src[0] + 8 * j;
    const int part = (8 * j) / P.C;
    return x + src[part] + (8 * j - part * P.C);
  };
  float s = 0.f, s2 = 0.f;
  for (int j = l16; j < nch; j += 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(chunk_ptr(j));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = bf_lo(v[p]), b2 = bf_hi(v[p]);
      s += a + b2;
      s2 = fmaf(a, a, fmaf(b2, b2, s2));
    }
  }
  s = sum16(s);
  s2 = sum16(s2);
  const float mean = s / Ct;
  const float var = fmaxf(s2 / Ct - mean * mean, 0.f);
  const float rstd = rsqrtf(var + P.eps);
  uint16_t* yo = y + t * Ct;
  for (int j = l16; j < nch; j += 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(chunk_ptr(j));
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * j);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * j + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(beta + 8 * j);
    const float4 b1 = *reinterpret_cast<const float4*>(beta + 8 * j + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = (bf_lo(v[p]) - mean) * rstd * gg[2 * p] + bb[2 * p];
      const float b2 = (bf_hi(v[p]) - mean) * rstd * gg[2 * p + 1] + bb[2 * p + 1];
      o[p] = pack_bf16(a, b2);
    }
    *reinterpret_cast<u32x4*>(yo + 8 * j) = o;
  }
}

// ---------------------------------------------------------------------------------------
// Overlapping stem: out[b][i][j][o] = bias[o] + sum_{c, di, dj} W[o][c][di][dj]
// img[b][p i + di - (p-1)][p j + dj - (p-1)][c], kernel k = 2p - 1, zero padding.  A thread
// computes 8 outputs of one token in fp32 from the weights staged in LDS as [tap][o].
// ---------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void wattn_stem_kernel(const uint16_t* __restrict__ img,
                                                         const uint16_t* __restrict__ W,
                                                         const float* __restrict__ bias,
                                                         uint16_t* __restrict__ y, const StemPlan P) {
  extern __shared__ float sW[];  // [k * k * Cin][Cout]
  const int k = 2 * P.p - 1, taps = k * k * P.Cin;
  for (int i = threadIdx.x; i < taps * P.Cout; i += blockDim.x) {
    // W is [Cout][Cin][k][k]; tap index = (di * k + dj) * Cin + c
    const int o = i / taps, r = i - o * taps;
    const int c = r / (k * k), rr = r - c * k * k;
    sW[(rr * P.Cin + c) * P.Cout + o] = __uint_as_float((uint32_t)W[i] << 16);
  }
  __syncthreads();
  const int groups = P.Cout / 8;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ntok = (int64_t)P.B * P.Ho * P.Wo;
  if (item >= ntok * groups) return;
  const int64_t tok = item / groups;
  const int og = (int)(item - tok * groups);
  const int64_t b = tok / ((int64_t)P.Ho * P.Wo);
  const int rem = (int)(tok - b * P.Ho * P.Wo);
  const int i = rem / P.Wo, j = rem - i * P.Wo;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = bias[8 * og + e];
  for (int di = 0; di < k; ++di) {
    const int yy = P.p * i + di - (P.p - 1);
    if (yy < 0 || yy >= P.Hi) continue;
    for (int dj = 0; dj < k; ++dj) {
      const int xx = P.p * j + dj - (P.p - 1);
      if (xx < 0 || xx >= P.Wi) continue;
      const uint16_t* px = img + ((b * P.Hi + yy) * P.Wi + xx) * P.Cin;
      for (int c = 0; c < P.Cin; ++c) {
        const float v = __uint_as_float((uint32_t)px[c] << 16);
        const float* w = &sW[((di * k + dj) * P.Cin + c) * P.Cout + 8 * og];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[e], v, acc[e]);
      }
    }
  }
  uint16_t* yo = y + tok * P.Cout + 8 * og;
  *reinterpret_cast<u32x4*>(yo) =
      u32x4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7])};
}

// Mean over the tokens of each image: y[b][c] = (1/n) sum_t x[b][t][c]; one thread per (b, c).
__global__ __launch_bounds__(256) void wattn_token_mean_kernel(const uint16_t* __restrict__ x,
                                                               uint16_t* __restrict__ y, int B, int n, int C) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * C) return;
  const int b = i / C, ch = i - b * C;
  const uint16_t* p = x + (int64_t)b * n * C + ch;
  float s = 0.f;
  for (int t = 0; t < n; ++t) s += __uint_as_float((uint32_t)p[(int64_t)t * C] << 16);
  y[i] = (uint16_t)(pack_bf16(s / n, 0.f) & 0xffffu);
}

}  // namespace

hipError_t wattn_launch_linear(const LinearPlan& P, int act, bool res, bool out_f32, const void* x, const void* W,
                               const float* bias, const void* r, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((P.M + 31) / 32), (unsigned)((P.N + 63) / 64));
  auto X = static_cast<const uint16_t*>(x);
  auto Wt = static_cast<const uint16_t*>(W);
  auto R = static_cast<const uint16_t*>(r);
#define WATTN_LIN(A, RS, F) \
  hipLaunchKernelGGL((wattn_linear_kernel<A, RS, F>), grid, dim3(64), 0, stream, X, Wt, bias, R, y, P)
  if (out_f32) {
    if (act != ACT_NONE || res) return hipErrorInvalidValue;
    WATTN_LIN(ACT_NONE, false, true);
  } else if (act == ACT_GELU) {
    if (res) return hipErrorInvalidValue;
    WATTN_LIN(ACT_GELU, false, false);
  } else if (res) {
    WATTN_LIN(ACT_NONE, true, false);
  } else {
    WATTN_LIN(ACT_NONE, false, false);
  }
#undef WATTN_LIN
  return hipGetLastError();
}

hipError_t wattn_launch_layernorm(const NormPlan& P, bool gather, const void* x, const float* gamma,
                                  const float* beta, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((P.T + 15) / 16));
  if (gather)
    hipLaunchKernelGGL((wattn_layernorm_kernel<true>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       gamma, beta, static_cast<uint16_t*>(y), P);
  else
    hipLaunchKernelGGL((wattn_layernorm_kernel<false>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), gamma, beta, static_cast<uint16_t*>(y), P);
  return hipGetLastError();
}

hipError_t wattn_launch_stem(const StemPlan& P, const void* img, const void* W, const float* bias, void* y,
                             hipStream_t stream) {
  const int k = 2 * P.p - 1;
  const size_t lds = (size_t)k * k * P.Cin * P.Cout * sizeof(float);
  const int64_t items = (int64_t)P.B * P.Ho * P.Wo * (P.Cout / 8);
  hipLaunchKernelGGL(wattn_stem_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), lds, stream,
                     static_cast<const uint16_t*>(img), static_cast<const uint16_t*>(W), bias,
                     static_cast<uint16_t*>(y), P);
  return hipGetLastError();
}

hipError_t wattn_launch_token_mean(const void* x, void* y, int B, int n, int C, hipStream_t stream) {
  hipLaunchKernelGGL(wattn_token_mean_kernel, dim3((unsigned)((B * C + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), B, n, C);
  return hipGetLastError();
}
