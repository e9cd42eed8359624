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
// A workgroup has C/32 waves and owns a strip of 16 columns and 16 output rows of one image.
// It slides down the strip with three input rows (with their halo columns) in LDS, loading
// each input row once and two rows ahead while the current row is computed.  Per output row:
//   depth-wise : each thread computes 8 channels of a token from the nine neighbouring tokens'
//                16-byte chunks in LDS (fp32 FMAs) and stores them to LDS as fp16;
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

constexpr int SW = 16;  // strip width (tokens per output row of a workgroup)
constexpr int SH = 16;  // output rows per workgroup

template <int C>
__global__ __launch_bounds__(2 * C) void wattn_cla_logits_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ w_dw,
                                                                 const float* __restrict__ b_dw,
                                                                 const float* __restrict__ w_pw,
                                                                 const float* __restrict__ b_pw,
                                                                 uint16_t* __restrict__ z, const ClaPlan P) {
  constexpr int NT = 2 * C;              // threads: C / 32 waves
  constexpr int CH = C / 8;              // 16-byte chunks per token
  constexpr int KS = C / 32;             // k steps of the point-wise product
  constexpr int YS = C + 8;              // LDS row stride (fp16) of the depth-wise tile
  constexpr int RW = SW + 2;             // input row width with the halo columns
  constexpr int RCH = RW * CH;           // 16-byte chunks of one input row
  constexpr int PF = (RCH + NT - 1) / NT;  // chunks per thread when a row is loaded
  // depth-wise weights as [tap][half][chunk][4] (channel 8 chunk + 4 half + e) and the bias as
  // [half][chunk][4]: the lanes of a wave read consecutive 16-byte words, free of bank conflicts
  __shared__ __align__(16) float sW[9 * C];
  __shared__ __align__(16) float sB[C];
  __shared__ __align__(16) uint16_t sX[3][RW * C];   // three input rows (bf16), rolling
  __shared__ __align__(16) uint16_t sY[SW * YS];     // depth-wise output of one row (fp16)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  // channel cidx = 8 chunk + 4 half + e sits at half * C/2 + 4 chunk + e of its tap's C floats
  auto wofs = [](int cidx) { return ((cidx >> 2) & 1) * (C / 2) + (cidx >> 3) * 4 + (cidx & 3); };
  for (int i = tid; i < 9 * C; i += NT) {  // w_dw is [C][3][3]
    const int cidx = i / 9, tap = i - cidx * 9;
    sW[tap * C + wofs(cidx)] = w_dw[i];
  }
  for (int i = tid; i < C; i += NT) sB[wofs(i)] = b_dw != nullptr ? b_dw[i] : 0.f;

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

  // this workgroup: image b, columns x0 .. x0 + SW - 1, output rows y0 .. y0 + SH - 1
  const int strips = (P.Wg + SW - 1) / SW, bands = (P.Hg + SH - 1) / SH;
  const int b = blockIdx.x / (strips * bands), rr = blockIdx.x - b * strips * bands;
  const int y0 = (rr / strips) * SH, x0 = (rr % strips) * SW;
  const int y1 = min(y0 + SH, P.Hg);
  const int64_t img = (int64_t)b * P.Hg * P.Wg;

  // input row yy (zero outside the image) as this thread's chunks of the RW x C row
  auto fetch_row = [&](int yy, u32x4 (&pre)[PF]) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = tid + f * NT;
      const int tx = it / CH, ch = it - tx * CH;
      const int xx = x0 - 1 + tx;
      const bool ok = it < RCH && yy >= 0 && yy < P.Hg && xx >= 0 && xx < P.Wg;
      pre[f] = ok ? *reinterpret_cast<const u32x4*>(x + (img + (int64_t)yy * P.Wg + xx) * C + 8 * ch)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_row = [&](int slot, const u32x4 (&pre)[PF]) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = tid + f * NT;
      if (it < RCH) *reinterpret_cast<u32x4*>(&sX[slot][it * 8]) = pre[f];
    }
  };
  auto slot_of = [](int yy) { return (yy + 3) % 3; };  // yy >= -1

  // one output row: rows y - 1 and y are in LDS; `pre` holds row y + 1 and is refilled with
  // row y + 3, so two rows are in flight while a row is computed
  auto do_row = [&](int y, u32x4 (&pre)[PF]) {
    store_row(slot_of(y + 1), pre);
    if (y + 3 <= y1) fetch_row(y + 3, pre);
    __syncthreads();
    // ---- depth-wise: SW tokens x CH chunks of 8 channels
    for (int it = tid; it < SW * CH; it += NT) {
      const int tx = it / CH, ch = it - tx * CH;
      const float4 b0 = *reinterpret_cast<const float4*>(&sB[4 * ch]);
      const float4 b1 = *reinterpret_cast<const float4*>(&sB[C / 2 + 4 * ch]);
      float acc[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int tap = 0; tap < 9; ++tap) {
        const int dy = tap / 3, dx = tap % 3;
        const u32x4 xr = *reinterpret_cast<const u32x4*>(&sX[slot_of(y - 1 + dy)][(tx + dx) * C + 8 * ch]);
        const float4 w0 = *reinterpret_cast<const float4*>(&sW[tap * C + 4 * ch]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sW[tap * C + C / 2 + 4 * ch]);
        acc[0] = fmaf(w0.x, bf_lo(xr[0]), acc[0]);
        acc[1] = fmaf(w0.y, bf_hi(xr[0]), acc[1]);
        acc[2] = fmaf(w0.z, bf_lo(xr[1]), acc[2]);
        acc[3] = fmaf(w0.w, bf_hi(xr[1]), acc[3]);
        acc[4] = fmaf(w1.x, bf_lo(xr[2]), acc[4]);
        acc[5] = fmaf(w1.y, bf_hi(xr[2]), acc[5]);
        acc[6] = fmaf(w1.z, bf_lo(xr[3]), acc[6]);
        acc[7] = fmaf(w1.w, bf_hi(xr[3]), acc[7]);
      }
      *reinterpret_cast<u32x4*>(&sY[tx * YS + 8 * ch]) =
          u32x4{pack_f16(acc[0], acc[1]), pack_f16(acc[2], acc[3]), pack_f16(acc[4], acc[5]), pack_f16(acc[6], acc[7])};
    }
    __syncthreads();
    // ---- point-wise: z^T[o][token] for this wave's 32 output channels, 16-token blocks
#pragma unroll
    for (int tb = 0; tb < SW / 16; ++tb) {
      const int tx = 16 * tb + c;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 Yf = *reinterpret_cast<const u32x4*>(&sY[tx * YS + 32 * ks + 8 * g]);
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) acc[ob] = mfma16_f16(Wf[ob][ks], Yf, acc[ob]);
      }
      if (x0 + tx < P.Wg) {
        const int64_t t = img + (int64_t)y * P.Wg + x0 + tx;
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) {
          const int o = 32 * wave + 16 * ob + 4 * g;
          *reinterpret_cast<u32x2*>(z + t * C + o) =
              u32x2{pack_bf16(acc[ob][0] + bias[ob][0], acc[ob][1] + bias[ob][1]),
                    pack_bf16(acc[ob][2] + bias[ob][2], acc[ob][3] + bias[ob][3])};
        }
      }
    }
  };

  u32x4 preA[PF], preB[PF];
  fetch_row(y0 - 1, preA);
  store_row(slot_of(y0 - 1), preA);
  fetch_row(y0, preA);
  store_row(slot_of(y0), preA);
  fetch_row(y0 + 1, preA);
  fetch_row(y0 + 2, preB);
  for (int y = y0; y < y1; y += 2) {
    do_row(y, preA);
    if (y + 1 < y1) do_row(y + 1, preB);
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
