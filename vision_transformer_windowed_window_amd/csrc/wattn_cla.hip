// wattn_cla.hip -- gate logits of the convolutional gate on the attention output (gfx950).
//
// Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution Transformer with
// FlashAttention, section 2.2: a 3x3 depth-wise and a 1x1 point-wise convolution of the layer
// input give a map that a sigmoid turns into the gate of the attention output.  This kernel
// computes the logits z = PW(DW3x3(x)); the sigmoid and the product with the attention output
// are fused into the attention kernel's epilogue.
//
//   x : [B][Hg][Wg][C] bf16 (channels last), w_dw [C][3][3], b_dw [C], w_pw [C][C] (out x in),
//   b_pw [C] fp32; z : [B][Hg][Wg][C] bf16.  Zero padding, stride 1, no activation between.
//
// A workgroup has C/32 waves and loops over tiles of 64 consecutive tokens (flattened
// b, y, x order).  Per tile:
//   depth-wise : each thread computes 8 channels of a token from the nine neighbouring tokens'
//                16-byte chunks (fp32 FMAs, weights from LDS) and stores them to LDS as fp16;
//   point-wise : z^T = W Y^T on 16x16x32 fp16 MFMA.  Wave w owns output channels
//                32 w .. 32 w + 31 and keeps their rows of W (fp16) in registers for the
//                whole kernel; the B operand (channels 8 g .. 8 g + 7 of token c) comes from the
//                LDS tile.  A lane's accumulator holds four consecutive output channels of one
//                token, stored as 8 bytes.
// fp16 operands limit |DW output| and |w_pw| to below 65504.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wattn_aux_plan.h"

namespace {

#include "wattn_device.h"

constexpr int CLA_TILE = 64;  // tokens per tile

template <int C>
__global__ __launch_bounds__(2 * C) void wattn_cla_logits_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ w_dw,
                                                                 const float* __restrict__ b_dw,
                                                                 const float* __restrict__ w_pw,
                                                                 const float* __restrict__ b_pw,
                                                                 uint16_t* __restrict__ z, const ClaPlan P) {
  constexpr int NT = 2 * C;            // threads: C / 32 waves
  constexpr int CH = C / 8;            // 16-byte chunks per token
  constexpr int KS = C / 32;           // k steps of the point-wise product
  constexpr int YS = C + 8;            // LDS row stride (fp16) of the tile, padded against bank conflicts
  __shared__ __align__(16) float sW[9 * C];   // depth-wise weights, [tap][channel]
  __shared__ __align__(16) float sB[C];       // depth-wise bias
  __shared__ __align__(16) uint16_t sY[CLA_TILE * YS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  for (int i = tid; i < 9 * C; i += NT) sW[(i % 9) * C + i / 9] = w_dw[i];  // [C][3][3] -> [tap][C]
  for (int i = tid; i < C; i += NT) sB[i] = b_dw != nullptr ? b_dw[i] : 0.f;

  // this wave's rows of W: output channels 32 wave + 16 ob + c, input channels 32 ks + 8 g .. + 7
  u32x4 Wf[2][KS];
  float bias[2][4];
#pragma unroll
  for (int ob = 0; ob < 2; ++ob) {
    const int o = 32 * wave + 16 * ob + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a0 = *reinterpret_cast<const float4*>(w_pw + (int64_t)o * C + 32 * ks + 8 * g);
      const float4 a1 = *reinterpret_cast<const float4*>(w_pw + (int64_t)o * C + 32 * ks + 8 * g + 4);
      Wf[ob][ks] = u32x4{pack_f16(a0.x, a0.y), pack_f16(a0.z, a0.w), pack_f16(a1.x, a1.y), pack_f16(a1.z, a1.w)};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) bias[ob][e] = b_pw != nullptr ? b_pw[32 * wave + 16 * ob + 4 * g + e] : 0.f;
  }
  __syncthreads();

  const int64_t ntok = (int64_t)P.B * P.Hg * P.Wg;
  const int64_t ntiles = (ntok + CLA_TILE - 1) / CLA_TILE;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * CLA_TILE;
    // ---- depth-wise: CLA_TILE * CH items of 8 channels.  The nine taps' loads are issued
    //      together from clamped (in-bounds) addresses; taps outside the grid get weight 0.
#pragma unroll 2
    for (int it = tid; it < CLA_TILE * CH; it += NT) {
      const int tl = it / CH, ch = it - tl * CH;
      const uint32_t t = (uint32_t)min(t0 + tl, ntok - 1);  // fewer than 2^31 tokens
      const uint32_t img = t / (uint32_t)(P.Hg * P.Wg);
      const uint32_t rem = t - img * (uint32_t)(P.Hg * P.Wg);
      const int yy = (int)(rem / (uint32_t)P.Wg), xx = (int)rem - yy * P.Wg;
      u32x4 xr[9];
      bool ok[9];
#pragma unroll
      for (int tap = 0; tap < 9; ++tap) {
        const int py = yy + tap / 3 - 1, px = xx + tap % 3 - 1;
        ok[tap] = py >= 0 && py < P.Hg && px >= 0 && px < P.Wg;
        const int cy = ok[tap] ? py : yy, cx = ok[tap] ? px : xx;
        xr[tap] = *reinterpret_cast<const u32x4*>(x + ((int64_t)(img * P.Hg + cy) * P.Wg + cx) * C + 8 * ch);
      }
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = sB[8 * ch + e];
#pragma unroll
      for (int tap = 0; tap < 9; ++tap) {
        const float* wt = &sW[tap * C + 8 * ch];
        const float4 w0 = *reinterpret_cast<const float4*>(wt);
        const float4 w1 = *reinterpret_cast<const float4*>(wt + 4);
        const float m = ok[tap] ? 1.0f : 0.0f;
        acc[0] = fmaf(w0.x * m, bf_lo(xr[tap][0]), acc[0]);
        acc[1] = fmaf(w0.y * m, bf_hi(xr[tap][0]), acc[1]);
        acc[2] = fmaf(w0.z * m, bf_lo(xr[tap][1]), acc[2]);
        acc[3] = fmaf(w0.w * m, bf_hi(xr[tap][1]), acc[3]);
        acc[4] = fmaf(w1.x * m, bf_lo(xr[tap][2]), acc[4]);
        acc[5] = fmaf(w1.y * m, bf_hi(xr[tap][2]), acc[5]);
        acc[6] = fmaf(w1.z * m, bf_lo(xr[tap][3]), acc[6]);
        acc[7] = fmaf(w1.w * m, bf_hi(xr[tap][3]), acc[7]);
      }
      *reinterpret_cast<u32x4*>(&sY[tl * YS + 8 * ch]) =
          u32x4{pack_f16(acc[0], acc[1]), pack_f16(acc[2], acc[3]), pack_f16(acc[4], acc[5]), pack_f16(acc[6], acc[7])};
    }
    __syncthreads();
    // ---- point-wise: per 16-token block, z^T[o][token] for this wave's 32 output channels
#pragma unroll
    for (int tb = 0; tb < CLA_TILE / 16; ++tb) {
      const int tl = 16 * tb + c;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 Yf = *reinterpret_cast<const u32x4*>(&sY[tl * YS + 32 * ks + 8 * g]);
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) acc[ob] = mfma16_f16(Wf[ob][ks], Yf, acc[ob]);
      }
      const int64_t t = t0 + tl;
      if (t < ntok) {
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) {
          const int o = 32 * wave + 16 * ob + 4 * g;
          *reinterpret_cast<u32x2*>(z + t * C + o) =
              u32x2{pack_bf16(acc[ob][0] + bias[ob][0], acc[ob][1] + bias[ob][1]),
                    pack_bf16(acc[ob][2] + bias[ob][2], acc[ob][3] + bias[ob][3])};
        }
      }
    }
    __syncthreads();  // the next tile overwrites sY
  }
}

template <int C>
hipError_t launch_cla(const ClaPlan& P, const void* x, const float* w_dw, const float* b_dw, const float* w_pw,
                      const float* b_pw, void* z, hipStream_t stream) {
  hipLaunchKernelGGL((wattn_cla_logits_kernel<C>), dim3(P.grid), dim3(2 * C), 0, stream,
                     static_cast<const uint16_t*>(x), w_dw, b_dw, w_pw, b_pw, static_cast<uint16_t*>(z), P);
  return hipGetLastError();
}

}  // namespace

hipError_t wattn_launch_cla(const ClaPlan& P, const void* x, const float* w_dw, const float* b_dw, const float* w_pw,
                            const float* b_pw, void* z, hipStream_t stream) {
  switch (P.C) {
    case 32: return launch_cla<32>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 64: return launch_cla<64>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 96: return launch_cla<96>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 128: return launch_cla<128>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 160: return launch_cla<160>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 192: return launch_cla<192>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 224: return launch_cla<224>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    case 256: return launch_cla<256>(P, x, w_dw, b_dw, w_pw, b_pw, z, stream);
    default: return hipErrorInvalidValue;
  }
}
