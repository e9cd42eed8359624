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
// The image is cut into column strips 16 tokens wide; the output rows of all strips, taken
// strip by strip, are split into equal runs, one per workgroup, with as many workgroups as the
// GPU holds at once (a run may finish one strip and continue at the top of the next).  A
// workgroup has C/32 waves.  It slides down its run with a ring of four input rows (with
// their halo columns) in LDS, loading each input row once, two rows before it is first
// needed.  Per output row:
//   depth-wise : thread t owns channels 2 j, 2 j + 1 (j = t mod C/2) of the four output
//                columns 4 q .. 4 q + 3 (q = t div C/2); it keeps those two channels' nine
//                taps in registers and reads the six input columns of each of the three rows
//                as 4-byte words (fp32 FMAs), then stores its four outputs to LDS as fp16;
//   point-wise : z^T = W Y^T on 16x16x32 fp16 MFMA.  Wave w owns output channels
//                32 w .. 32 w + 31 and keeps their rows of W (fp16) in registers for the
//                whole kernel; the B operand (channels 8 g .. 8 g + 7 of token c) comes from the
//                LDS tile.  A lane's accumulator holds four consecutive output channels of one
//                token, stored as 8 bytes.
// The depth-wise tile is double-buffered and the input ring has a spare row, so one barrier per
// output row orders every LDS hazard.
// fp16 operands limit |DW output| and |w_pw| to below 65504.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "wattn_aux_plan.h"

namespace {

#include "wattn_device.h"

constexpr int SW = 16;  // strip width (tokens per output row of a workgroup)

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
  static_assert(NT == (C / 2) * (SW / 4), "one depth-wise item per thread");
  __shared__ __align__(16) uint16_t sX[4][RW * C];   // ring of four input rows (bf16)
  __shared__ __align__(16) uint16_t sY[2][SW * YS];  // depth-wise output of a row (fp16), double-buffered

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  // this workgroup's run: rows r_begin .. r_end - 1 of the strip-major row sequence (strip
  // `col` = b * strips + column block, row y); the current segment is rows y0 .. y1 - 1 of image
  // b, columns x0 .. x0 + SW - 1
  const int strips = (P.Wg + SW - 1) / SW;
  int r = blockIdx.x * P.per;  // below rows: the grid is ceil(rows / per)
  const int r_end = (int)min((int64_t)P.rows, (int64_t)r + P.per);
  int b, x0, y0, y1;
  int64_t img;
  auto set_segment = [&]() {
    const int col = r / P.Hg;
    y0 = r - col * P.Hg;
    b = col / strips;
    x0 = (col - b * strips) * SW;
    y1 = min(P.Hg, y0 + (r_end - r));
    img = (int64_t)b * P.Hg * P.Wg;
  };
  set_segment();

  // input row yy as this thread's chunks of the RW x C row.  Every load is issued, from a
  // clamped in-bounds address, and `ok` records which chunks lie inside the image: the zero
  // padding is applied when the row is stored to LDS.  Loads that are never skipped keep the
  // row loop free of branches around memory operations, so the compiler can wait for exactly
  // the row that is needed instead of for every load in flight.
  auto fetch_row = [&](int yy, u32x4 (&pre)[PF], uint32_t& ok) {
    ok = 0;
    const int yc = min(max(yy, 0), P.Hg - 1);
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = min(tid + f * NT, RCH - 1);
      const int tx = it / CH, ch = it - tx * CH;
      const int xx = x0 - 1 + tx;
      const int xc = min(max(xx, 0), P.Wg - 1);
      ok |= (yy >= 0 && yy < P.Hg && xx >= 0 && xx < P.Wg) ? (1u << f) : 0u;
      pre[f] = *reinterpret_cast<const u32x4*>(x + (img + (int64_t)yc * P.Wg + xc) * C + 8 * ch);
    }
  };
  auto store_row = [&](int yy, const u32x4 (&pre)[PF], uint32_t ok) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = tid + f * NT;
      const u32x4 v = (ok >> f) & 1u ? pre[f] : u32x4{0u, 0u, 0u, 0u};
      if (it < RCH) *reinterpret_cast<u32x4*>(&sX[(yy + 4) & 3][it * 8]) = v;
    }
  };

  // the first three input rows go out before the weights, so their latency overlaps the
  // weight loads
  u32x4 preA[PF], preB[PF], preC[PF];
  uint32_t okA, okB, okC;
  fetch_row(y0 - 1, preA, okA);
  fetch_row(y0, preB, okB);
  fetch_row(y0 + 1, preC, okC);

  // ---- depth-wise item of this thread: channels 2 jc, 2 jc + 1 of output columns 4 qc .. 4 qc + 3
  const int jc = tid % (C / 2), qc = tid / (C / 2);
  float wd[9][2], bd[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int tap = 0; tap < 9; ++tap) wd[tap][e] = w_dw[(2 * jc + e) * 9 + tap];
    bd[e] = b_dw != nullptr ? b_dw[2 * jc + e] : 0.f;
  }

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

  // One output row y.  Rows y - 1 .. y + 1 are in the ring; `pre` holds row y + 2, which goes
  // into the ring slot row y - 2 held, and is refilled with row y + 4.  Hazards: that slot was
  // last read by row y - 1's depth-wise step and sY[y & 1] by row y - 2's point-wise step, both
  // before the previous row's barrier.
  auto do_row = [&](int y, u32x4 (&pre)[PF], uint32_t& ok) {
    store_row(y + 2, pre, ok);  // rows past y1 are never read
    fetch_row(y + 4, pre, ok);
    uint16_t* Y = sY[y & 1];
    {
      float acc[4][2];
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        acc[o][0] = bd[0];
        acc[o][1] = bd[1];
      }
#pragma unroll
      for (int dy = 0; dy < 3; ++dy) {
        const uint16_t* row = &sX[(y - 1 + dy + 4) & 3][(4 * qc) * C + 2 * jc];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const uint32_t xv = *reinterpret_cast<const uint32_t*>(row + i * C);
          const float x0v = bf_lo(xv), x1v = bf_hi(xv);
#pragma unroll
          for (int o = 0; o < 4; ++o) {
            const int dx = i - o;
            if (dx >= 0 && dx < 3) {
              acc[o][0] = fmaf(wd[3 * dy + dx][0], x0v, acc[o][0]);
              acc[o][1] = fmaf(wd[3 * dy + dx][1], x1v, acc[o][1]);
            }
          }
        }
      }
#pragma unroll
      for (int o = 0; o < 4; ++o)
        *reinterpret_cast<uint32_t*>(&Y[(4 * qc + o) * YS + 2 * jc]) = pack_f16(acc[o][0], acc[o][1]);
    }
    __syncthreads();
    // ---- point-wise: z^T[o][token] for this wave's 32 output channels, 16-token blocks
#pragma unroll
    for (int tb = 0; tb < SW / 16; ++tb) {
      const int tx = 16 * tb + c;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 Yf = *reinterpret_cast<const u32x4*>(&Y[tx * YS + 32 * ks + 8 * g]);
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) acc[ob] = mfma16_f16(Wf[ob][ks], Yf, acc[ob]);
      }
      // z through a buffer resource spanning this row from column x0 to the image edge: a
      // token past the edge has an offset beyond the resource, and the hardware drops its
      // store.  No branch around the stores, so the row loop's waits count them exactly.
      const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
          z + (img + (int64_t)y * P.Wg + x0) * C, 0, (P.Wg - x0) * C * 2, 0x00020000);
#pragma unroll
      for (int ob = 0; ob < 2; ++ob) {
        const int o = 32 * wave + 16 * ob + 4 * g;
        const u32x2 v = {pack_bf16(acc[ob][0] + bias[ob][0], acc[ob][1] + bias[ob][1]),
                         pack_bf16(acc[ob][2] + bias[ob][2], acc[ob][3] + bias[ob][3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, rz, (tx * C + o) * 2, 0, 0);
      }
    }
  };

  const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc(z, 0, 0, 0x00020000);
  while (true) {
    store_row(y0 - 1, preA, okA);
    store_row(y0, preB, okB);
    store_row(y0 + 1, preC, okC);
    // Two stores that the hardware drops (a resource of zero bytes) follow each prefetch, so
    // that the row loop is entered with the same memory operations in flight as on later
    // iterations (a row's loads, then its two z stores): the compiler's count of younger
    // operations at each wait is then exact on every path.  They only make the compiler's
    // waits tight, not correct: every load here goes to registers, which the compiler tracks,
    // so an added or removed memory operation can lengthen a wait but never shorten it below
    // what the data needs.
    fetch_row(y0 + 2, preA, okA);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rnone, 0, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rnone, 64, 0, 0);
    fetch_row(y0 + 3, preB, okB);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rnone, 0, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rnone, 64, 0, 0);
    __syncthreads();
    int y = y0;
    for (; y + 1 < y1; y += 2) {  // no exit between the two rows: the waits stay exact
      do_row(y, preA, okA);
      do_row(y + 1, preB, okB);
    }
    if (y < y1) do_row(y, preA, okA);
    r += y1 - y0;
    if (r >= r_end) break;
    // the run continues at the top of the next strip: the ring and the depth-wise tiles are
    // refilled once every wave is done with them
    set_segment();
    fetch_row(y0 - 1, preA, okA);
    fetch_row(y0, preB, okB);
    fetch_row(y0 + 1, preC, okC);
    __syncthreads();
  }
}

template <int C>
hipError_t launch_cla(ClaPlan P, const void* x, const float* w_dw, const float* b_dw, const float* w_pw,
                      const float* b_pw, void* z, hipStream_t stream) {
  // as many workgroups as the GPU holds at once, each with an equal run of rows
  static int slots_cache[16] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int slots = dev < 16 ? __atomic_load_n(&slots_cache[dev], __ATOMIC_RELAXED) : 0;
  if (slots == 0) {
    int per_cu = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wattn_cla_logits_kernel<C>, 2 * C, 0)) !=
        hipSuccess)
      return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    slots = std::max(1, per_cu) * std::max(1, cus);
    if (dev < 16) __atomic_store_n(&slots_cache[dev], slots, __ATOMIC_RELAXED);
  }
  P.per = (P.rows + slots - 1) / slots;
  P.grid = (P.rows + P.per - 1) / P.per;
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
