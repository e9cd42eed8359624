// wattn_gated.hip -- device code of the gated local path of libwattn.so for gfx950.
//
// HSMLA: Hierarchical Softmax Multi-scale Linear Attention for Efficient Vision Transformers,
// technical summary section 2 (method).  A gate shared by all heads scores each spatial
// block; the blocks whose gate exceeds a threshold tau take a local softmax path inside a
// small w x w window, and their output becomes the global (ReLU linear attention) output plus
// the residual R = O_local - O_lin-local.  The page asks that routing work on whole tiles
// (contiguous memory, no per-token divergence) and that the selected tiles run as a compacted
// pipeline; here:
//
//   wattn_select_blocks_kernel : one workgroup compacts the indices of the blocks with
//       gate > tau into an ascending list (wave ballots and a prefix over the waves).
//   wattn_local_residual_kernel : one workgroup per (listed block, head), the grid sized for
//       every block and the workgroups past the device-side count leaving at once; or, in
//       the one-launch form, one workgroup per (block, head) of the grid that leaves unless
//       the block's gate exceeds tau.  The
//       block's K and V (at most 16 x 16 tokens) are staged whole in LDS; each wave owns 16
//       queries and computes
//         O_local      exact softmax over the block's keys: S^T = K Q^T on bf16 MFMA (bf16
//                      products are exact in the fp32 accumulator), the exact row max from
//                      the scores held in registers, P = 2^((s - max) log2(e) / sqrt(d))
//                      rounded to fp16 (P <= 1), O^T += V^T P^T on fp16 MFMA;
//         O_lin-local  relu(q)^T KV / (relu(q) . ksum + eps) with KV = sum_j relu(k_j) v_j^T
//                      and ksum = sum_j relu(k_j) built once per block on bf16 MFMA (the key
//                      sums as a product with a ones operand), kept in fp32 in LDS and fed to
//                      the apply product as a bf16 high part plus a bf16 low part;
//       and adds O_local - O_lin-local to `out` in place (fp32, one rounding to the output
//       type at the end).
//
// V is staged twice: bf16 for the KV product and fp16 for the value product.  fp16 holds
// magnitudes below 65504, so v entries must stay below that.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wattn_aux_plan.h"

namespace {

#include "wattn_device.h"

typedef short i16x2 __attribute__((ext_vector_type(2)));

// max(x, 0) of two packed bf16: a bf16 is negative exactly when its bit pattern, read as a
// 16-bit integer, is negative (-0 included), so an integer max with 0 clears it.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  const i16x2 s = __builtin_bit_cast(i16x2, w);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(s, i16x2{0, 0}));
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

__global__ __launch_bounds__(1024) void wattn_select_blocks_kernel(const float* __restrict__ gate, int n, float tau,
                                                                   int* __restrict__ list, int* __restrict__ count) {
  __shared__ int sCnt[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += 1024) {
    const int i = i0 + tid;
    const bool sel = i < n && gate[i] > tau;  // NaN compares false
    const uint64_t m = __ballot(sel);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) sCnt[wave] = __popcll(m);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int cw = sCnt[w];
      pre += w < wave ? cw : 0;
      tot += cw;
    }
    if (sel) list[base + pre + below] = i;
    base += tot;
    __syncthreads();  // sCnt is rewritten by the next chunk
  }
  if (tid == 0) *count = base;
}

// LISTED: the blocks come from a list and its device-side count (wattn_select_blocks);
// otherwise every block of the grid has a workgroup per head that routes itself by reading
// the block's gate (one launch, no list).
template <int W, bool OUTF32, bool LISTED>
__global__ __launch_bounds__(64 * ((W * W + 15) / 16)) void wattn_local_residual_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ out, const int* __restrict__ list, const int* __restrict__ count,
    const float* __restrict__ gate, float tau, const LocalPlan P) {
  constexpr int T = W * W;                 // queries = keys of a block
  constexpr int KP = (T + 31) / 32 * 32;   // keys padded to whole 32-key steps (zero rows)
  constexpr int NWV = (T + 15) / 16;       // waves, 16 queries each
  constexpr int NT = 64 * NWV;
  constexpr int NKB = KP / 16;             // 16-key score blocks
  constexpr int KVS = 36;                  // LDS row stride (floats) of the [dim][channel] KV matrix
  __shared__ __align__(16) uint16_t sK[KP * D];   // bf16
  __shared__ __align__(16) uint16_t sVb[KP * D];  // bf16
  __shared__ __align__(16) uint16_t sVh[KP * D];  // fp16
  __shared__ __align__(16) float sKV[D * KVS];    // [dim][channel]: sum_j relu(k_j)[ch] v_j[dim]
  __shared__ __align__(16) float sKS[D];          // sum_j relu(k_j)[ch]

  // ---- task: (entry i, head h).  Workgroups are dealt to the 8 XCDs round-robin; workgroup
  //      x + 8 r (x < 8) takes entry x + 8 (r / H) and head r % H, so the heads of a block,
  //      whose rows share cache lines, meet in one XCD's L2.  An entry is a list position
  //      (LISTED: entries past the count and entries outside the grid are skipped) or a block
  //      (its gate must exceed tau; a NaN gate does not).
  const int xr = blockIdx.x >> 3;
  const int i = (blockIdx.x & 7) + 8 * (xr / P.H), h = xr - (xr / P.H) * P.H;
  int blk;
  if (LISTED) {
    const int listed = min(max(*count, 0), P.nblocks);
    if (i >= listed) return;
    blk = list[i];
    if (blk < 0 || blk >= P.nblocks) return;
  } else {
    if (i >= P.nblocks || !(gate[i] > tau)) return;
    blk = i;
  }
  const int b = blk / P.nW, rb = blk - b * P.nW;
  const int wy = rb / P.nWx, wx = rb - wy * P.nWx;
  const int y0 = wy * W, x0 = wx * W;
  const int64_t hbase = (int64_t)b * P.img_stride + h * D;
  const int tokstride = P.H * D;
  auto tok_off = [&](int n) -> int64_t {
    return hbase + ((int64_t)(y0 + n / W) * P.Wg + (x0 + n % W)) * tokstride;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- stage the block's K and V (16-byte chunk tid % 4 of key row tid / 4)
  for (int row = tid >> 2; row < KP; row += NT / 4) {
    const int ch = tid & 3;
    u32x4 kk = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u}, vh = {0u, 0u, 0u, 0u};
    if (row < T) {
      const int64_t o = tok_off(row) + 8 * ch;
      kk = *reinterpret_cast<const u32x4*>(k + o);
      vb = *reinterpret_cast<const u32x4*>(v + o);
#pragma unroll
      for (int p = 0; p < 4; ++p) vh[p] = pack_f16(bf_lo(vb[p]), bf_hi(vb[p]));
    }
    *reinterpret_cast<u32x4*>(&sK[row * D + ((ch ^ kswz(row)) * 8)]) = kk;
    *reinterpret_cast<u32x4*>(&sVb[row * D + ((ch ^ vswz(row)) * 8)]) = vb;
    *reinterpret_cast<u32x4*>(&sVh[row * D + ((ch ^ vswz(row)) * 8)]) = vh;
  }
  // this wave's queries (query c of the wave, channels 8 g .. 8 g + 7): the B operand of the
  // score product, and with negative channels cleared, of the linear product
  const int qn = wave * 16 + c;
  const bool qvalid = qn < T;
  u32x4 Qf = {0u, 0u, 0u, 0u};
  // the lane's part of `out` (dims 16 db + 4 g .. + 3 of query qn), read now so that the
  // read's latency passes while the block is computed
  f32x4 base[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  u32x2 base16[2] = {{0u, 0u}, {0u, 0u}};
  const int64_t qoff = tok_off(qn);
  if (qvalid) {
    Qf = *reinterpret_cast<const u32x4*>(q + qoff + 8 * g);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      if (OUTF32)
        base[db] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(out) + qoff + 16 * db + 4 * g);
      else
        base16[db] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(out) + qoff + 16 * db + 4 * g);
    }
  }
  __syncthreads();

  // transposed-read coordinates: lane (c, g) of a 32-key step reads keys 8 g + (c >> 2) and
  // 8 g + (c >> 2) + 4, 16-byte chunk (c & 3) >> 1 of the 32-byte half, 8-byte part c & 1
  const int vrow = 8 * g + (c >> 2);
  const int vch = (c & 3) >> 1, vsub = 4 * (c & 1);
  // score rows: row c of 16-key block 2 s + b reads key 32 s + 8 (c >> 2) + (c & 3) + 4 b, so a
  // lane's accumulator rows are keys 32 s + 8 g + 4 b + e: eight consecutive keys per step
  const int krow = 8 * (c >> 2) + (c & 3);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // ---- KV = relu(K)^T V and ksum = relu(K)^T 1: six 16x16 jobs dealt to the waves
  for (int job = wave; job < 6; job += NWV) {
    const int cb = job < 4 ? (job >> 1) : job - 4;  // channel block
    const int db = job & 1;                         // dim block (KV jobs)
    f32x4 acc = zero;
#pragma unroll
    for (int ks = 0; ks < KP / 32; ++ks) {
      u32x2 hk[2], hv[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 32 * ks + vrow + 4 * hh;
        hk[hh] = lds_read_tr16(&sK[row * D + (((2 * cb + vch) ^ kswz(row)) * 8) + vsub]);
        hv[hh] = lds_read_tr16(&sVb[row * D + (((2 * db + vch) ^ vswz(row)) * 8) + vsub]);
      }
      // A: relu(k)^T, row = channel 16 cb + c, k = keys 8 g .. 8 g + 7 of the step
      const u32x4 KT = {relu_bf16x2(hk[0][0]), relu_bf16x2(hk[0][1]), relu_bf16x2(hk[1][0]), relu_bf16x2(hk[1][1])};
      // B: v (column = dim 16 db + c) or ones
      const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
      const u32x4 VB = job < 4 ? u32x4{hv[0][0], hv[0][1], hv[1][0], hv[1][1]} : ones;
      acc = mfma16_bf16(KT, VB, acc);
    }
    // lane (c, g) holds rows (channels) 16 cb + 4 g + e of column c
    if (job < 4) {
      *reinterpret_cast<f32x4*>(&sKV[(16 * db + c) * KVS + 16 * cb + 4 * g]) = acc;
    } else if (c == 0) {
      *reinterpret_cast<f32x4*>(&sKS[16 * cb + 4 * g]) = acc;
    }
  }

  // ---- O_local: scores of all keys, exact row max, P in fp16, O^T = V^T P^T
  f32x4 S[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = 32 * (kb >> 1) + krow + 4 * (kb & 1);
    const u32x4 Kf = *reinterpret_cast<const u32x4*>(&sK[key * D + ((g ^ kswz(key)) * 8)]);
    S[kb] = mfma16_bf16(Kf, Qf, zero);
  }
  if (T % 32 != 0) {  // padded keys of the last step
#pragma unroll
    for (int kb = NKB - 2; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + e >= T) S[kb][e] = -INFINITY;
  }
  float m = S[0][0];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, S[kb][e]);
  m = xmax32(xmax16(m));
  constexpr float SC = LOG2E * 0.17677669529663687f;  // log2(e) / sqrt(32)
  const float msc = -m * SC;
  const u32x4 ONE16 = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
  f32x4 O[2] = {zero, zero};  // [dim block]: dims 16 db + 4 g + e of query c
  float l = 0.f;
#pragma unroll
  for (int s = 0; s < KP / 32; ++s) {
    uint32_t Pw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = 2 * s + (t >> 1), e0 = 2 * (t & 1);
      Pw[t] = pack_f16(__builtin_amdgcn_exp2f(fmaf(S[kb][e0], SC, msc)),
                       __builtin_amdgcn_exp2f(fmaf(S[kb][e0 + 1], SC, msc)));
      l = dot2_f16(Pw[t], ONE16[0], l);  // the row sum of the rounded weights
    }
    const u32x4 Pa = {Pw[0], Pw[1], Pw[2], Pw[3]};
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      u32x2 hv[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 32 * s + vrow + 4 * hh;
        hv[hh] = lds_read_tr16(&sVh[row * D + (((2 * db + vch) ^ vswz(row)) * 8) + vsub]);
      }
      O[db] = mfma16_f16(u32x4{hv[0][0], hv[0][1], hv[1][0], hv[1][1]}, Pa, O[db]);
    }
  }
  l = xsum32(xsum16(l));
  __syncthreads();  // KV and ksum complete

  // ---- O_lin-local = relu(q)^T KV / (relu(q) . ksum + eps)
  const u32x4 Qr = {relu_bf16x2(Qf[0]), relu_bf16x2(Qf[1]), relu_bf16x2(Qf[2]), relu_bf16x2(Qf[3])};
  float den = 0.f;
  {
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(&sKS[8 * g]);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(&sKS[8 * g + 4]);
    den = fmaf(bf_lo(Qr[0]), k0[0], den);
    den = fmaf(bf_hi(Qr[0]), k0[1], den);
    den = fmaf(bf_lo(Qr[1]), k0[2], den);
    den = fmaf(bf_hi(Qr[1]), k0[3], den);
    den = fmaf(bf_lo(Qr[2]), k1[0], den);
    den = fmaf(bf_hi(Qr[2]), k1[1], den);
    den = fmaf(bf_lo(Qr[3]), k1[2], den);
    den = fmaf(bf_hi(Qr[3]), k1[3], den);
  }
  den = xsum32(xsum16(den)) + P.eps;
  f32x4 Num[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    // A: row = dim 16 db + c, k = channels 8 g .. 8 g + 7, as bf16 high and low parts
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sKV[(16 * db + c) * KVS + 8 * g]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sKV[(16 * db + c) * KVS + 8 * g + 4]);
    const float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    u32x4 hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      hi[p] = pack_bf16(x[2 * p], x[2 * p + 1]);
      lo[p] = pack_bf16(x[2 * p] - bf_lo(hi[p]), x[2 * p + 1] - bf_hi(hi[p]));
    }
    Num[db] = mfma16_bf16(hi, Qr, zero);
    Num[db] = mfma16_bf16(lo, Qr, Num[db]);
  }

  // ---- out += O_local - O_lin-local (dims 16 db + 4 g .. + 3 of query qn)
  if (qvalid) {
    const float il = 1.0f / l, iden = 1.0f / den;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = O[db][e] * il - Num[db][e] * iden;
      if (OUTF32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + qoff + 16 * db + 4 * g) =
            f32x4{base[db][0] + r[0], base[db][1] + r[1], base[db][2] + r[2], base[db][3] + r[3]};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + qoff + 16 * db + 4 * g) =
            u32x2{pack_bf16(bf_lo(base16[db][0]) + r[0], bf_hi(base16[db][0]) + r[1]),
                  pack_bf16(bf_lo(base16[db][1]) + r[2], bf_hi(base16[db][1]) + r[3])};
      }
    }
  }
}

template <int W, bool LISTED>
hipError_t launch_local_w(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v, void* out,
                          const int* list, const int* count, const float* gate, float tau, hipStream_t stream) {
  constexpr int NT = 64 * ((W * W + 15) / 16);
  const dim3 grid((unsigned)(8 * P.H * ((P.nblocks + 7) / 8)));
  const uint16_t *q16 = static_cast<const uint16_t*>(q), *k16 = static_cast<const uint16_t*>(k),
                 *v16 = static_cast<const uint16_t*>(v);
  if (out_f32)
    hipLaunchKernelGGL((wattn_local_residual_kernel<W, true, LISTED>), grid, dim3(NT), 0, stream, q16, k16, v16,
                       out, list, count, gate, tau, P);
  else
    hipLaunchKernelGGL((wattn_local_residual_kernel<W, false, LISTED>), grid, dim3(NT), 0, stream, q16, k16, v16,
                       out, list, count, gate, tau, P);
  return hipGetLastError();
}

template <bool LISTED>
hipError_t launch_local(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v, void* out,
                        const int* list, const int* count, const float* gate, float tau, hipStream_t stream) {
  switch (P.w) {
    case 4: return launch_local_w<4, LISTED>(P, out_f32, q, k, v, out, list, count, gate, tau, stream);
    case 8: return launch_local_w<8, LISTED>(P, out_f32, q, k, v, out, list, count, gate, tau, stream);
    case 12: return launch_local_w<12, LISTED>(P, out_f32, q, k, v, out, list, count, gate, tau, stream);
    case 16: return launch_local_w<16, LISTED>(P, out_f32, q, k, v, out, list, count, gate, tau, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t wattn_launch_select(const float* gate, int n, float tau, int* list, int* count, hipStream_t stream) {
  hipLaunchKernelGGL(wattn_select_blocks_kernel, dim3(1), dim3(1024), 0, stream, gate, n, tau, list, count);
  return hipGetLastError();
}

hipError_t wattn_launch_local(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v,
                              void* out, const int* list, const int* count, hipStream_t stream) {
  return launch_local<true>(P, out_f32, q, k, v, out, list, count, nullptr, 0.f, stream);
}

hipError_t wattn_launch_gated(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v,
                              void* out, const float* gate, float tau, hipStream_t stream) {
  return launch_local<false>(P, out_f32, q, k, v, out, nullptr, nullptr, gate, tau, stream);
}
