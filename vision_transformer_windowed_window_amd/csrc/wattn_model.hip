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

#include "wattn_aux_plan.h"

namespace {

#include "wattn_device.h"

// ---------------------------------------------------------------------------------------
// y = act(x W^T + b) (+ res).  A workgroup of 4 waves computes a tile of 128 tokens x 128
// outputs, the waves as 2 x 2 sub-tiles of 64 x 64, as y^T = W x^T on 16x16x32 bf16 MFMA: A =
// 16 rows of W, B = 16 tokens of x, 8 consecutive inputs per lane.  The 32-wide k slices of x
// and W go from global memory straight into LDS (16 bytes per lane, no registers), three slices
// in flight: the slice two steps ahead is requested while the current one is multiplied.  A
// slice row is 64 bytes; chunk j of row r sits in LDS slot j ^ ((r >> 2) & 3), so that the 16
// rows a fragment read touches fall on distinct banks (the loads fetch the swizzled chunk, as
// the LDS position of a lane's data is fixed by its lane index).  Each wave reads 4 + 4
// fragments per slice for 16 MFMAs.  A lane's accumulator holds four consecutive outputs of one
// token, stored as 8 bytes.  Output column n goes to part n / split at offset
// part * part_stride + m * split + n % split, which writes q, k and v of a qkv projection as
// three separate [M][C] tensors.
// ---------------------------------------------------------------------------------------

enum { ACT_NONE = 0, ACT_GELU = 1 };

// GELU(x) = 0.5 x (1 + erf(x / sqrt 2)).  With z = |x| / sqrt 2, 1 + erf(x / sqrt 2) is
// erfc(z) for x < 0 and 2 - erfc(z) for x >= 0, and erfc(z) = t exp(-z^2 + P(t)) with
// t = 1 / (1 + z / 2) and P of degree 7 fitted by csrc/fit_erfc.py (relative error of erfc
// below 6.4e-7 in exact arithmetic; the float32 evaluation here adds rounding up to about 2e-5
// of erfc where -z^2 is large).  Hardware reciprocal and exp2.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = -1.836619680e-01f;
  p = fmaf(p, t, 7.339941066e-01f);
  p = fmaf(p, t, -9.701263864e-01f);
  p = fmaf(p, t, 3.209165196e-01f);
  p = fmaf(p, t, -2.418480100e-02f);
  p = fmaf(p, t, 3.892575659e-01f);
  p = fmaf(p, t, 9.993278403e-01f);
  p = fmaf(p, t, -1.265523516e+00f);
  const float q = t * __builtin_amdgcn_exp2f(fmaf(-z, z, p) * 1.4426950408889634f);
  return 0.5f * x * (x >= 0.f ? 2.0f - q : q);
}

constexpr int LT = 128;     // tile rows (tokens) and columns (outputs)
constexpr int LSTAGE = 3;   // k slices in flight
constexpr int LSL = LT * 32;  // bf16 elements of one operand's slice
// Direct-to-LDS loads per k slice and wave: LT / 64 = 2 instructions (64 rows of 16-byte
// chunks each) for each of the two operands.  The main loop's hand-written wait leaves exactly
// one slice's loads in flight, so it counts these and nothing else: the loop must issue no
// other vector-memory instruction (the epilogue's loads and stores come after it).
constexpr int LIN_LOAD_HALVES = LT / 64;
constexpr int LIN_SLICE_LOADS = 2 * LIN_LOAD_HALVES;

__device__ __forceinline__ int lswz(int row) { return (row >> 2) & 3; }

template <int ACT, bool RES, bool OUTF32>
__global__ __launch_bounds__(256) void wattn_linear_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ W,
                                                           const float* __restrict__ bias,
                                                           const uint16_t* res, void* y, const LinearPlan P) {
  __shared__ __align__(16) uint16_t sS[LSTAGE][2][LSL];  // [stage][x, W][row * 32 + swizzled chunk * 8]
  __shared__ float sBias[LT];  // bias of the tile's outputs (0 past N or without a bias)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  // workgroups are dealt to the 8 XCDs round-robin: workgroup x + 8 r (x < 8) takes m tile
  // x + 8 (r / ntn) and n tile r % ntn, so the n tiles of one m tile (which share its rows of
  // x) run one after another in the same XCD's L2
  const int ntn = (P.N + LT - 1) / LT;
  const int xr = blockIdx.x >> 3;
  const int mt = (blockIdx.x & 7) + 8 * (xr / ntn), nt = xr - (xr / ntn) * ntn;
  if (mt * LT >= P.M) return;
  const int m0 = mt * LT, n0 = nt * LT;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;  // this wave's sub-tile
  // loads: instruction h of wave w fills LDS chunks 256 h + 64 w + lane of a slice, i.e. row
  // 64 h + 16 w + lane / 4, slot lane % 4, from the chunk that the swizzle puts there; rows
  // past M (N) reload the last row, whose products are never stored
  const uint16_t* xs[LIN_LOAD_HALVES];
  const uint16_t* ws[LIN_LOAD_HALVES];
#pragma unroll
  for (int h = 0; h < LIN_LOAD_HALVES; ++h) {
    const int row = 64 * h + 16 * wave + (lane >> 2), chunk = (lane & 3) ^ lswz(row);
    xs[h] = x + (int64_t)min(m0 + row, P.M - 1) * P.K + 8 * chunk;
    ws[h] = W + (int64_t)min(n0 + row, P.N - 1) * P.K + 8 * chunk;
  }
  auto issue = [&](int ks, int stage) {  // LIN_SLICE_LOADS vector-memory instructions, no more
#pragma unroll
    for (int h = 0; h < LIN_LOAD_HALVES; ++h) {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(xs[h] + 32 * ks),
                                       (__attribute__((address_space(3))) void*)(&sS[stage][0][(256 * h + 64 * wave) * 8]),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ws[h] + 32 * ks),
                                       (__attribute__((address_space(3))) void*)(&sS[stage][1][(256 * h + 64 * wave) * 8]),
                                       16, 0, 0);
    }
  };
  f32x4 acc[4][4];  // [n block][m block]
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = P.K / 32;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  // (waits for the slices issued above too, as they are older: step 0 needs slice 0 anyway)
  if (tid < LT) sBias[tid] = (bias != nullptr && n0 + tid < P.N) ? bias[n0 + tid] : 0.f;
  // The compiler orders LDS reads after direct-to-LDS loads by waiting for every load in
  // flight, which would drain the pipeline each step; the barrier and the fragment reads are
  // therefore written out, with the waits they need and no more.
  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks % LSTAGE;
    // this wave's loads of slice ks are done when at most slice ks + 1's four loads are still in
    // flight; the barrier then covers every wave's loads (and, on the first step, sBias)
    if (ks + 1 < nk)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LIN_SLICE_LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // slice ks + 2 goes into the stage slice ks - 1 used, which every wave finished reading
    // (its reads end with a wait) before the barrier above
    if (ks + 2 < nk) issue(ks + 2, (ks + 2) % LSTAGE);
    // fragments: rows wn + 16 i + c of W and wm + 16 i + c of x, chunk g (swizzled); the
    // reads complete inside the statement, so their registers are written when it ends
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&sS[stage][0][0];
    const uint32_t ax = base + (uint32_t)((wm + c) * 64 + 16 * (g ^ lswz(wm + c)));
    const uint32_t aw = base + (uint32_t)(LSL * 2 + (wn + c) * 64 + 16 * (g ^ lswz(wn + c)));
    u32x4 af[4], bfr[4];
    // the swizzle of row base + 16 i + c is that of row c ((row >> 2) & 3, and 16 i and the
    // sub-tile bases 0 and 64 add multiples of 4 to row >> 2), so fragment i is 1024 bytes
    // (16 rows of 64 bytes) past fragment 0
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:1024\n\t"
        "ds_read_b128 %6, %9 offset:2048\n\t"
        "ds_read_b128 %7, %9 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bfr[0]), "=&v"(bfr[1]), "=&v"(bfr[2]),
          "=&v"(bfr[3])  // early clobber: a read may land before the next one takes its address
        : "v"(aw), "v"(ax)
        : "memory");
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma16_bf16(af[nb], bfr[mb], acc[nb][mb]);
  }
  // epilogue: lane (c, g) holds outputs n0 + wn + 16 nb + 4 g + e of token m0 + wm + 16 mb + c.
  // The bias comes from LDS; the four residual words of a token block are loaded together, from
  // clamped in-bounds addresses (N is a multiple of 4), so that one wait covers them.
  auto out_off = [&](int m, int n) {
    const int part = n / P.split, nn = n - part * P.split;
    return (int64_t)part * P.part_stride + (int64_t)m * P.split + nn;
  };
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm + 16 * mb + c;
    if (m >= P.M) continue;
    u32x2 rv[4];
    if (RES) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        rv[nb] = *reinterpret_cast<const u32x2*>(res + out_off(m, min(n0 + wn + 16 * nb + 4 * g, P.N - 4)));
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn + 16 * nb + 4 * g;
      if (n >= P.N) continue;
      const int64_t off = out_off(m, n);
      const float4 bv = *reinterpret_cast<const float4*>(&sBias[wn + 16 * nb + 4 * g]);
      float r[4] = {acc[nb][mb][0] + bv.x, acc[nb][mb][1] + bv.y, acc[nb][mb][2] + bv.z, acc[nb][mb][3] + bv.w};
      if (ACT == ACT_GELU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = gelu_erf(r[e]);
      }
      if (RES) {
        r[0] += bf_lo(rv[nb][0]);
        r[1] += bf_hi(rv[nb][0]);
        r[2] += bf_lo(rv[nb][1]);
        r[3] += bf_hi(rv[nb][1]);
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

// The same for rows of at most 16 * CPL chunks (the normalised width of the model's norms is at
// most 1536): each lane keeps its CPL chunks of the row in registers between the two passes,
// and the workgroup stages gamma and beta in LDS.  Every row load is issued (a lane past the
// row's chunks reloads the last chunk and zeroes it), before the gain and bias loads, so one
// memory latency covers them all.
constexpr int LN_MAXC = 1536;

template <bool GATHER, int CPL>
__global__ __launch_bounds__(256) void wattn_layernorm_reg_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ gamma,
                                                                  const float* __restrict__ beta,
                                                                  uint16_t* __restrict__ y, const NormPlan P) {
  __shared__ __align__(16) float sG[LN_MAXC];
  __shared__ __align__(16) float sBt[LN_MAXC];
  const int tid = threadIdx.x, l16 = tid & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 16 + (tid >> 4);  // output token
  const bool valid = t0 < P.T;
  const int64_t t = valid ? t0 : P.T - 1;
  const int Ct = GATHER ? 4 * P.C : P.C;  // channels of the normalised row
  const int nch = Ct / 8;
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
  u32x4 xr[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) xr[i] = *reinterpret_cast<const u32x4*>(chunk_ptr(min(l16 + 16 * i, nch - 1)));
  for (int i = tid; i < Ct; i += 256) {
    sG[i] = gamma[i];
    sBt[i] = beta[i];
  }
  float s = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (l16 + 16 * i >= nch) xr[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = bf_lo(xr[i][p]), b2 = bf_hi(xr[i][p]);
      s += a + b2;
      s2 = fmaf(a, a, fmaf(b2, b2, s2));
    }
  }
  s = sum16(s);
  s2 = sum16(s2);
  const float mean = s / Ct;
  const float var = fmaxf(s2 / Ct - mean * mean, 0.f);
  const float rstd = rsqrtf(var + P.eps);
  __syncthreads();  // sG, sBt
  if (!valid) return;
  uint16_t* yo = y + t * Ct;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int j = l16 + 16 * i;
    if (j >= nch) break;
    const float4 g0 = *reinterpret_cast<const float4*>(&sG[8 * j]);
    const float4 g1 = *reinterpret_cast<const float4*>(&sG[8 * j + 4]);
    const float4 b0 = *reinterpret_cast<const float4*>(&sBt[8 * j]);
    const float4 b1 = *reinterpret_cast<const float4*>(&sBt[8 * j + 4]);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = (bf_lo(xr[i][p]) - mean) * rstd * gg[2 * p] + bb[2 * p];
      const float b2 = (bf_hi(xr[i][p]) - mean) * rstd * gg[2 * p + 1] + bb[2 * p + 1];
      o[p] = pack_bf16(a, b2);
    }
    *reinterpret_cast<u32x4*>(yo + 8 * j) = o;
  }
}

// ---------------------------------------------------------------------------------------
// Overlapping stem: out[b][i][j][o] = bias[o] + sum_{c, di, dj} W[o][c][di][dj]
// img[b][p i + di - (p-1)][p j + dj - (p-1)][c], kernel k = 2p - 1, zero padding.  A thread
// computes 32 outputs of one token in fp32; the weights sit in LDS as [tap][Cout], so the
// threads of a wave that share an output slice read the same LDS words (broadcast).
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
  const int groups = P.Cout / 32;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ntok = (int64_t)P.B * P.Ho * P.Wo;
  if (item >= ntok * groups) return;
  const int64_t tok = item / groups;
  const int og = (int)(item - tok * groups);
  const int64_t b = tok / ((int64_t)P.Ho * P.Wo);
  const int rem = (int)(tok - b * P.Ho * P.Wo);
  const int i = rem / P.Wo, j = rem - i * P.Wo;
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = bias[32 * og + e];
  for (int di = 0; di < k; ++di) {
    const int yy = P.p * i + di - (P.p - 1);
    if (yy < 0 || yy >= P.Hi) continue;
    for (int dj = 0; dj < k; ++dj) {
      const int xx = P.p * j + dj - (P.p - 1);
      if (xx < 0 || xx >= P.Wi) continue;
      const uint16_t* px = img + ((b * P.Hi + yy) * P.Wi + xx) * P.Cin;
      for (int c = 0; c < P.Cin; ++c) {
        const float v = __uint_as_float((uint32_t)px[c] << 16);
        const float4* w = reinterpret_cast<const float4*>(&sW[((di * k + dj) * P.Cin + c) * P.Cout + 32 * og]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 wq = w[q];
          acc[4 * q] = fmaf(wq.x, v, acc[4 * q]);
          acc[4 * q + 1] = fmaf(wq.y, v, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(wq.z, v, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(wq.w, v, acc[4 * q + 3]);
        }
      }
    }
  }
  uint16_t* yo = y + tok * P.Cout + 32 * og;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4*>(yo + 8 * q) =
        u32x4{pack_bf16(acc[8 * q], acc[8 * q + 1]), pack_bf16(acc[8 * q + 2], acc[8 * q + 3]),
              pack_bf16(acc[8 * q + 4], acc[8 * q + 5]), pack_bf16(acc[8 * q + 6], acc[8 * q + 7])};
}

// Mean over the tokens of each image: y[b][c] = (1/n) sum_t x[b][t][c].  A workgroup owns 64
// channels of one image: thread t sums the 8 channels of chunk t % 8 over tokens t / 8,
// t / 8 + 32, ...; the 32 partial sums per channel meet in LDS.
__global__ __launch_bounds__(256) void wattn_token_mean_kernel(const uint16_t* __restrict__ x,
                                                               uint16_t* __restrict__ y, int B, int n, int C) {
  __shared__ float part[32][65];
  const int tid = threadIdx.x, ch = tid & 7, row = tid >> 3;
  const int b = blockIdx.y, c0 = blockIdx.x * 64 + 8 * ch;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < C) {
    const uint16_t* p = x + (int64_t)b * n * C + c0;
    for (int t = row; t < n; t += 32) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + (int64_t)t * C);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[2 * q] += bf_lo(v[q]);
        s[2 * q + 1] += bf_hi(v[q]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[row][8 * ch + e] = s[e];
  __syncthreads();
  if (tid < 64 && blockIdx.x * 64 + tid < C) {
    float t = 0.f;
    for (int r = 0; r < 32; ++r) t += part[r][tid];
    y[(int64_t)b * C + blockIdx.x * 64 + tid] = (uint16_t)(pack_bf16(t / n, 0.f) & 0xffffu);
  }
}

}  // namespace

hipError_t wattn_launch_linear(const LinearPlan& P, int act, bool res, bool out_f32, const void* x, const void* W,
                               const float* bias, const void* r, void* y, hipStream_t stream) {
  const int64_t mtiles = (P.M + LT - 1) / LT, ntiles = (P.N + LT - 1) / LT;
  const dim3 grid((unsigned)(8 * ntiles * ((mtiles + 7) / 8)));
  auto X = static_cast<const uint16_t*>(x);
  auto Wt = static_cast<const uint16_t*>(W);
  auto R = static_cast<const uint16_t*>(r);
#define WATTN_LIN(A, RS, F) \
  hipLaunchKernelGGL((wattn_linear_kernel<A, RS, F>), grid, dim3(256), 0, stream, X, Wt, bias, R, y, P)
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

template <bool G>
static hipError_t launch_layernorm_g(const NormPlan& P, const void* x, const float* gamma, const float* beta, void* y,
                                     hipStream_t stream) {
  const dim3 grid((unsigned)((P.T + 15) / 16));
  auto X = static_cast<const uint16_t*>(x);
  auto Y = static_cast<uint16_t*>(y);
  const int Ct = G ? 4 * P.C : P.C;
  const int cpl = (Ct / 8 + 15) / 16;  // chunks per lane
#define WATTN_LN(K) hipLaunchKernelGGL(K, grid, dim3(256), 0, stream, X, gamma, beta, Y, P)
  if (Ct > LN_MAXC) WATTN_LN((wattn_layernorm_kernel<G>));
  else if (cpl <= 1) WATTN_LN((wattn_layernorm_reg_kernel<G, 1>));
  else if (cpl <= 2) WATTN_LN((wattn_layernorm_reg_kernel<G, 2>));
  else if (cpl <= 3) WATTN_LN((wattn_layernorm_reg_kernel<G, 3>));
  else if (cpl <= 6) WATTN_LN((wattn_layernorm_reg_kernel<G, 6>));
  else WATTN_LN((wattn_layernorm_reg_kernel<G, 12>));
#undef WATTN_LN
  return hipGetLastError();
}

hipError_t wattn_launch_layernorm(const NormPlan& P, bool gather, const void* x, const float* gamma,
                                  const float* beta, void* y, hipStream_t stream) {
  return gather ? launch_layernorm_g<true>(P, x, gamma, beta, y, stream)
                : launch_layernorm_g<false>(P, x, gamma, beta, y, stream);
}

hipError_t wattn_launch_stem(const StemPlan& P, const void* img, const void* W, const float* bias, void* y,
                             hipStream_t stream) {
  const int k = 2 * P.p - 1;
  const size_t lds = (size_t)k * k * P.Cin * P.Cout * sizeof(float);
  const int64_t items = (int64_t)P.B * P.Ho * P.Wo * (P.Cout / 32);
  hipLaunchKernelGGL(wattn_stem_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), lds, stream,
                     static_cast<const uint16_t*>(img), static_cast<const uint16_t*>(W), bias,
                     static_cast<uint16_t*>(y), P);
  return hipGetLastError();
}

hipError_t wattn_launch_token_mean(const void* x, void* y, int B, int n, int C, hipStream_t stream) {
  hipLaunchKernelGGL(wattn_token_mean_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)B), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), B, n, C);
  return hipGetLastError();
}
