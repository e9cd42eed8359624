// wattn_kernels.hip -- device code of libwattn.so for gfx950 (AMD Instinct MI355X).
//
// Fused shifted-window attention (FLASHSWIN page, "How it works", first and second
// changes; RIB page, section 2.1 for the bias channels).
//
// Work decomposition.  A shifted window of the last row or column band holds two (corner:
// four) wrap regions; tokens attend only within their region, and each region is a
// rectangle of tokens that is contiguous in the ORIGINAL (un-shifted) grid.  A workgroup
// of 8 waves owns 256 queries (32 per wave) of one region of one window and head and
// streams the region's keys through LDS in tiles of 64.  The masked pairs of the shifted
// layer are never computed.
//
//   prologue : decode the task; build the window-local cos/sin table of the head in LDS
//              (fp32 angles, hardware sin/cos); each wave loads its 32 queries straight
//              from their original positions, rotates them in fp32, folds in
//              d^-1/2 * log2(e), rounds once to fp16 and keeps them in registers; with a
//              bias, u * log2(e) is appended as 16 more channels.
//   key loop : per tile, threads 0..255 fetch one 16-byte chunk of K each and threads
//              256..511 one chunk of V (and of the bias factor v) for the next tile while
//              the current tile is computed; then K is rotated in fp32, rounded to fp16
//              and stored with V (bf16, unchanged) into the other LDS buffer (both
//              row-major, chunk-swizzled against bank conflicts).  Per 32-key step each
//              wave runs
//                  S^T = K Q^T        32x32x16 fp16 MFMA, accumulator preset to -m,
//                  p   = 2^(S^T)      fp32 online softmax in registers,
//                  O^T += V^T P^T     32x32x16 bf16 MFMA, V^T read with ds_read_tr16_b64.
//              The transposed products keep each query's scores, running max m, running
//              sum l and output column in one lane (the lane pair l, l^32 splits the keys).
//   epilogue : O / l, stored as bf16 (round to nearest even) or fp32 at the tokens'
//              original positions, which reverses the cyclic shift.
//
// The running max is updated lazily: with the accumulator preset to -m, S^T already holds
// s - m and p = 2^(s - m) costs one exp per score.  The exact rescale (row max, O and l
// scaled by 2^-delta) runs for the first key step and whenever some p of a step exceeds
// 2^16, so every p stays within [0, 2^16] (row sums stay below 2^16 * N).  Row sums are
// taken over the bf16-rounded p that the PV product consumes.
//
// Precision: q, k, v arrive in bf16 and RoPE runs in fp32 (FLASHSWIN page, closing
// developer paragraph).  The rotated, scaled q and k are rounded once to fp16 (11-bit
// significand) for the score product: rounding them to bf16 (8-bit significand) instead
// moves logits by up to ~1e-2 relative and alone costs up to 1e-2 absolute in the output
// on N(0,1) workloads.  fp16 limits the score operands to |value| < 65504; larger q, k or
// bias-factor entries overflow and give non-finite outputs.  P is rounded to bf16 for the
// PV product (P can reach 2^16, beyond fp16).
//
// The fp32 path (wattn_fwd_f32_kernel) is a plain per-query loop over the whole window
// with the region-label mask, used for float32 inputs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wattn_plan.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 32;          // head dimension of q, k, v
constexpr int NTHR = 512;      // threads per workgroup of the bf16 path (8 waves)
constexpr int QT = WATTN_BF16_QTILE;  // queries per workgroup (32 per wave)
constexpr int KT = 64;         // keys per LDS tile
constexpr int MAXM = 128;      // largest window side (cos/sin table rows)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LIMIT = 65536.0f;  // 2^16

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f32x2 f = {a, b};
  f16x2 h = __builtin_convertvector(f, f16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// score product: fp16 operands, fp32 accumulate
__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// value product: bf16 operands, fp32 accumulate
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed 8-byte LDS read (gfx950): in each group of 16 lanes, lane j receives element
// j % 4 of the 8-byte reads issued by lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// i / den and i % den for 0 <= i < 2^16 and 1 <= den <= 2^16, via a multiply-high.
struct Divider {
  uint32_t den, magic;
  __device__ explicit Divider(uint32_t d) : den(d), magic(d == 1 ? 0u : 0xffffffffu / d + 1u) {}
  __device__ __forceinline__ void split(uint32_t i, int& qt, int& rm) const {
    const uint32_t qq = (den == 1) ? i : __umulhi(i, magic);
    qt = (int)qq;
    rm = (int)(i - qq * den);
  }
};

// Chunk swizzles (16-byte chunks of a 64-byte K or V row).  K: the eight rows that one
// MFMA operand read touches per LDS cycle land in eight distinct bank groups.  V: the four
// rows of one transposed read group land in distinct bank halves / chunk pairs.
__device__ __forceinline__ int kswz(int key) { return ((key >> 1) & 1) | (((key >> 4) & 1) << 1); }
__device__ __forceinline__ int vswz(int key) { return ((key >> 1) & 1) << 1; }

// Row of the K tile that feeds MFMA A-operand row i (0..31): the accumulator row layout of
// the 32x32 MFMA then gives lane (query, g) the scores of keys 16g .. 16g+15 in order.
__device__ __forceinline__ int key_of_row(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

struct Task {
  int b, h, q0;
  int r0, rh, c0, rw;  // region in window-local coordinates
  int y0, x0;          // region origin in the original grid (the region does not wrap)
};

// Workgroup bid -> task.  Consecutive groups of `chunk` tasks go to one XCD (workgroups
// are dealt to the 8 XCDs round-robin), so tasks that share cache lines meet in one L2.
__device__ __forceinline__ bool decode_task(const WattnPlan& P, int bid, Task& t) {
  const int C = P.chunk;
  const int xcd = bid & 7, slot = bid >> 3;
  const int task = ((slot / C) * 8 + xcd) * C + (slot % C);
  if (task >= P.ntasks) return false;
  WattnSeg S = P.seg[0];
#pragma unroll
  for (int i = 1; i < WATTN_MAX_SEG; ++i)
    if (i < P.nseg && task >= P.seg[i].task_begin) S = P.seg[i];
  int u = task - S.task_begin;
  const int qt = u % S.nqt;
  u /= S.nqt;
  t.h = u % P.H;
  u /= P.H;
  const int nw = S.nwy * S.nwx;
  const int wi = u % nw;
  t.b = u / nw;
  const int wy = S.wy0 + wi / S.nwx;
  const int wx = S.wx0 + wi % S.nwx;
  t.r0 = S.r0;
  t.rh = S.rh;
  t.c0 = S.c0;
  t.rw = S.rw;
  t.q0 = qt * QT;
  int y = wy * P.M + S.r0 + P.s;
  if (y >= P.Hg) y -= P.Hg;
  int x = wx * P.M + S.c0 + P.s;
  if (x >= P.Wg) x -= P.Wg;
  t.y0 = y;
  t.x0 = x;
  return true;
}

template <int NKS, bool ROPE, bool OUTF32>
__global__ __launch_bounds__(NTHR) void wattn_fwd_bf16_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              void* __restrict__ out,
                                                              const float* __restrict__ theta,
                                                              const uint16_t* __restrict__ bu,
                                                              const uint16_t* __restrict__ bv,
                                                              const WattnPlan P) {
  constexpr bool BIAS = (NKS == 3);
  __shared__ __align__(16) uint16_t sK[2][KT * D];
  __shared__ __align__(16) uint16_t sV[2][KT * D];
  __shared__ __align__(16) uint16_t sKb[BIAS ? 2 : 1][BIAS ? KT * 16 : 8];
  __shared__ float2 sTab[ROPE ? MAXM * (D / 2) : 1];

  Task T;
  if (!decode_task(P, blockIdx.x, T)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = P.M;
  const int h = T.h;
  const int n = T.rh * T.rw;
  const int colstride = P.H * D;            // elements between horizontally adjacent tokens
  const int rowstride = P.Wg * colstride;   // elements between vertically adjacent tokens
  const int64_t img = (int64_t)T.b * P.Hg * rowstride;
  const int regbase = T.y0 * rowstride + T.x0 * colstride + h * D;
  const uint16_t* qi_ = q + img;
  const uint16_t* ki_ = k + img;
  const uint16_t* vi_ = v + img;
  const Divider div(T.rw);

  if (ROPE) {
    for (int i = tid; i < M * (D / 2); i += NTHR) {
      const int pos = i >> 4, j = i & 15;
      float sn, cs;
      __sincosf((float)pos * theta[h * (D / 2) + j], &sn, &cs);
      sTab[i] = make_float2(cs, sn);
    }
    __syncthreads();
  }

  const int qi = lane & 31, g = lane >> 5;
  const bool wave_live = T.q0 + wave * 32 < n;  // wave-uniform

  // ---- queries: rotate in fp32, scale by d^-1/2 * log2(e), round once to fp16
  u32x4 Qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) Qf[ks] = u32x4{0u, 0u, 0u, 0u};
  {
    const int iq = T.q0 + wave * 32 + qi;
    const float qscale = LOG2E * 0.17677669529663687f;  // log2(e) / sqrt(32)
    if (iq < n) {
      int li, lj;
      div.split((uint32_t)iq, li, lj);
      const int off = regbase + li * rowstride + lj * colstride;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(qi_ + off + 16 * ks + 8 * g);
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float a = bf_lo(raw[p]), c = bf_hi(raw[p]);
          if (ROPE) {
            const int pos = (ks == 0) ? (T.r0 + li) : (T.c0 + lj);
            const float2 t = sTab[pos * (D / 2) + 8 * ks + 4 * g + p];
            const float a2 = a * t.x - c * t.y;
            const float c2 = a * t.y + c * t.x;
            a = a2;
            c = c2;
          }
          o[p] = pack_f16(a * qscale, c * qscale);
        }
        Qf[ks] = o;
      }
      if (BIAS) {
        const int nl = (T.r0 + li) * M + (T.c0 + lj);
        const u32x4 raw = *reinterpret_cast<const u32x4*>(bu + ((int64_t)h * M * M + nl) * 16 + 8 * g);
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = pack_f16(bf_lo(raw[p]) * LOG2E, bf_hi(raw[p]) * LOG2E);
        Qf[NKS - 1] = o;
      }
    }
  }

  // ---- loader: threads 0..255 own a K chunk (key lk, channels 8*lch..), 256..511 the V
  //      chunk; threads 256..383 also own a bias-factor chunk (key bk, channels 8*bch..).
  //      The key index advances by KT per tile; region coordinates and the element offset
  //      are carried along incrementally.
  const bool kthread = tid < 256;
  const int lk = (tid & 255) >> 2, lch = tid & 3;
  const int bk = (tid & 127) >> 1, bch = tid & 1;
  const bool bthread = BIAS && tid >= 256 && tid < 384;
  const int step_i = KT / T.rw, step_j = KT % T.rw;
  const int step_off = step_i * rowstride + step_j * colstride;  // offset change without carry
  const int carry_off = rowstride - T.rw * colstride;              // extra change on a column carry
  int ci, cj, bi, bj;
  div.split((uint32_t)lk, ci, cj);
  div.split((uint32_t)bk, bi, bj);
  int koff = regbase + ci * rowstride + cj * colstride + 8 * lch;  // element offset of the chunk
  const uint16_t* ksrc = (kthread ? ki_ : vi_);
  const uint16_t* bsrc = bv + (int64_t)h * M * M * 16 + 8 * bch;
  u32x4 pd = {0u, 0u, 0u, 0u}, pb = {0u, 0u, 0u, 0u};
  int lpos = 0;

  auto advance = [&]() {
    ci += step_i;
    cj += step_j;
    koff += step_off;
    if (cj >= T.rw) {
      cj -= T.rw;
      ci += 1;
      koff += carry_off;
    }
    if (BIAS) {
      bi += step_i;
      bj += step_j;
      if (bj >= T.rw) {
        bj -= T.rw;
        bi += 1;
      }
    }
  };
  auto fetch = [&](int tile) {
    pd = u32x4{0u, 0u, 0u, 0u};
    if (tile * KT + lk < n) {
      pd = *reinterpret_cast<const u32x4*>(ksrc + koff);
      lpos = (lch < 2) ? (T.r0 + ci) : (T.c0 + cj);
    }
    if (BIAS) {
      pb = u32x4{0u, 0u, 0u, 0u};
      if (bthread && tile * KT + bk < n)
        pb = *reinterpret_cast<const u32x4*>(bsrc + ((T.r0 + bi) * M + (T.c0 + bj)) * 16);
    }
  };
  auto store = [&](int buf) {
    if (kthread) {
      u32x4 kr;
      if (ROPE) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float a = bf_lo(pd[p]), c = bf_hi(pd[p]);
          const float2 t = sTab[lpos * (D / 2) + 4 * lch + p];
          kr[p] = pack_f16(a * t.x - c * t.y, a * t.y + c * t.x);
        }
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) kr[p] = pack_f16(bf_lo(pd[p]), bf_hi(pd[p]));
      }
      *reinterpret_cast<u32x4*>(&sK[buf][lk * D + ((lch ^ kswz(lk)) * 8)]) = kr;
    } else {
      *reinterpret_cast<u32x4*>(&sV[buf][lk * D + ((lch ^ vswz(lk)) * 8)]) = pd;
    }
    if (BIAS && bthread) {
      u32x4 br;
#pragma unroll
      for (int p = 0; p < 4; ++p) br[p] = pack_f16(bf_lo(pb[p]), bf_hi(pb[p]));
      *reinterpret_cast<u32x4*>(&sKb[buf][bk * 16 + ((bch ^ ((bk >> 4) & 1)) * 8)]) = br;
    }
  };

  // ---- per-query online-softmax state (lane = query; lanes l and l^32 hold the same m)
  f32x16 O, Cn;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    O[e] = 0.f;
    Cn[e] = 0.f;
  }
  float m = 0.f, l = 0.f;
  const uint32_t ONES = 0x3f803f80u;  // bf16 pair (1.0, 1.0)
  const int ntile = (n + KT - 1) / KT;

  // per-lane constants of the operand reads
  const int arow = key_of_row(lane & 31);             // K tile row feeding A-operand row lane%32
  const int vgrp = lane >> 4;                         // 16-lane group of the transposed V read
  const int vs = lane & 15;                           // source lane within the group
  const int vchunk_hi = (vgrp & 1) * 2;               // dims 0..15 -> chunks 0,1; 16..31 -> 2,3

  fetch(0);
  store(0);
  advance();
  __syncthreads();

#pragma unroll 2
  for (int tile = 0; tile < ntile; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntile) fetch(tile + 1);

    if (wave_live) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kb = st * 32;
        const int kg = tile * KT + kb;  // first key of the step (uniform)
        if (kg < n) {
          const int key = kb + arow;
          u32x4 Kf[NKS];
          Kf[0] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + (((0 + g) ^ kswz(key)) * 8)]);
          Kf[1] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + (((2 + g) ^ kswz(key)) * 8)]);
          if (BIAS)
            Kf[NKS - 1] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 16 + ((g ^ ((key >> 4) & 1)) * 8)]);
          // V^T operand of the two PV MFMAs: keys kb + 16g + 8j + 4u + t, dims of this lane
          u32x2 Vt[2][2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int row = kb + 16 * (vgrp >> 1) + 8 * j + 4 * u + (vs >> 2);
              const int chunk = vchunk_hi + ((vs & 3) >> 1);
              Vt[j][u] = lds_read_tr16(&sV[buf][row * D + ((chunk ^ vswz(row)) * 8) + 4 * (vs & 1)]);
            }

          f32x16 S = mfma32_f16(Kf[0], Qf[0], Cn);
#pragma unroll
          for (int ks = 1; ks < NKS; ++ks) S = mfma32_f16(Kf[ks], Qf[ks], S);
          if (kg + 32 > n) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (kg + 16 * g + e >= n) S[e] = -INFINITY;
          }
          const bool first = (tile == 0) && (st == 0);
          uint32_t Pp[8];
          float ls = 0.f;
          bool exact = first;
          if (!first) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              Pp[t] = pack_bf16(__builtin_amdgcn_exp2f(S[2 * t]), __builtin_amdgcn_exp2f(S[2 * t + 1]));
              ls = dot2_bf16(Pp[t], ONES, ls);
            }
            exact = __any(ls > RESCALE_LIMIT);
          }
          if (exact) {
            float mx = S[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float delta = first ? mx : fmaxf(mx, 0.f);
            if (!first) {
              const float a = __builtin_amdgcn_exp2f(-delta);
              l *= a;
#pragma unroll
              for (int e = 0; e < 16; ++e) O[e] *= a;
            }
            m += delta;
#pragma unroll
            for (int e = 0; e < 16; ++e) Cn[e] = -m;
            ls = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              Pp[t] = pack_bf16(__builtin_amdgcn_exp2f(S[2 * t] - delta),
                                __builtin_amdgcn_exp2f(S[2 * t + 1] - delta));
              ls = dot2_bf16(Pp[t], ONES, ls);
            }
          }
          l += ls;
          const u32x4 P0 = {Pp[0], Pp[1], Pp[2], Pp[3]};
          const u32x4 P1 = {Pp[4], Pp[5], Pp[6], Pp[7]};
          O = mfma32(u32x4{Vt[0][0][0], Vt[0][0][1], Vt[0][1][0], Vt[0][1][1]}, P0, O);
          O = mfma32(u32x4{Vt[1][0][0], Vt[1][0][1], Vt[1][1][0], Vt[1][1][1]}, P1, O);
        }
      }
    }

    if (tile + 1 < ntile) {
      store(buf ^ 1);
      advance();
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, scatter to the original positions
  const float lt = l + __shfl_xor(l, 32);
  const int iq = T.q0 + wave * 32 + qi;
  if (iq < n) {
    const float inv = 1.0f / lt;
    int li, lj;
    div.split((uint32_t)iq, li, lj);
    const int64_t off = img + regbase + li * rowstride + lj * colstride;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (OUTF32) {
        const float4 w = make_float4(O[4 * t + 0] * inv, O[4 * t + 1] * inv, O[4 * t + 2] * inv, O[4 * t + 3] * inv);
        *reinterpret_cast<float4*>(static_cast<float*>(out) + off + 8 * t + 4 * g) = w;
      } else {
        u32x2 w;
        w[0] = pack_bf16(O[4 * t + 0] * inv, O[4 * t + 1] * inv);
        w[1] = pack_bf16(O[4 * t + 2] * inv, O[4 * t + 3] * inv);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + off + 8 * t + 4 * g) = w;
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// fp32 path: one thread per query, whole window, explicit region-label mask.
// ------------------------------------------------------------------------------------

__device__ __forceinline__ int axis_label(int P, int G, int M, int s) {
  if (s == 0 || P < G - M) return 0;
  return (P < G - s) ? 1 : 2;
}

template <int R>
__global__ __launch_bounds__(256) void wattn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, float* __restrict__ out,
                                                            const float* __restrict__ theta,
                                                            const float* __restrict__ bu,
                                                            const float* __restrict__ bv, const WattnF32Plan P) {
  constexpr int FK = 64;  // keys per LDS tile
  __shared__ float sK[FK][D + R + 1];
  __shared__ float sV[FK][D];
  __shared__ int sLab[FK];
  __shared__ float2 sTab[MAXM * (D / 2)];

  int u = blockIdx.x;
  const int qt = u % P.nqt;
  u /= P.nqt;
  const int h = u % P.H;
  u /= P.H;
  const int w = u % P.nw;
  const int b = u / P.nw;
  const int wy = w / P.nwx, wx = w % P.nwx;
  const int M = P.M, N = M * M, s = P.s;
  const int tid = threadIdx.x;
  const bool rope = theta != nullptr;

  if (rope) {
    for (int i = tid; i < M * (D / 2); i += 256) {
      const int pos = i >> 4, j = i & 15;
      double sn, cs;
      sincos((double)pos * (double)theta[h * (D / 2) + j], &sn, &cs);
      sTab[i] = make_float2((float)cs, (float)sn);
    }
  }
  __syncthreads();

  auto offset = [&](int lr, int lc) -> int64_t {
    int y = wy * M + lr + s;
    if (y >= P.Hg) y -= P.Hg;
    int x = wx * M + lc + s;
    if (x >= P.Wg) x -= P.Wg;
    return ((((int64_t)b * P.Hg + y) * P.Wg + x) * P.H + h) * D;
  };

  const int iq = qt * 256 + tid;
  const bool valid = iq < N;
  const int qr = valid ? iq / M : 0, qc = valid ? iq % M : 0;
  const int qlab = axis_label(wy * M + qr, P.Hg, M, s) * 3 + axis_label(wx * M + qc, P.Wg, M, s);
  float qv[D], uq[R > 0 ? R : 1], o[D];
  const float scale = 0.17677669529663687f;  // 1/sqrt(32)
  if (valid) {
    const float* src = q + offset(qr, qc);
#pragma unroll
    for (int j = 0; j < D / 2; ++j) {
      float a = src[2 * j], c = src[2 * j + 1];
      if (rope) {
        const float2 t = sTab[((j < D / 4) ? qr : qc) * (D / 2) + j];
        const float a2 = a * t.x - c * t.y, c2 = a * t.y + c * t.x;
        a = a2;
        c = c2;
      }
      qv[2 * j] = a * scale;
      qv[2 * j + 1] = c * scale;
    }
    if (R > 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) uq[t] = bu[((int64_t)h * N + iq) * R + t];
    }
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) qv[j] = 0.f;
#pragma unroll
    for (int t = 0; t < (R > 0 ? R : 1); ++t) uq[t] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < D; ++j) o[j] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int k0 = 0; k0 < N; k0 += FK) {
    const int kc = min(FK, N - k0);
    // load: thread -> (key tid/4, 8 channels)
    {
      const int kk = tid >> 2, ch = tid & 3;
      if (kk < kc) {
        const int key = k0 + kk;
        const int kr = key / M, kcc = key % M;
        const int64_t off = offset(kr, kcc);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int j = 4 * ch + p;
          float a = k[off + 2 * j], c = k[off + 2 * j + 1];
          if (rope) {
            const float2 t = sTab[((j < D / 4) ? kr : kcc) * (D / 2) + j];
            const float a2 = a * t.x - c * t.y, c2 = a * t.y + c * t.x;
            a = a2;
            c = c2;
          }
          sK[kk][2 * j] = a;
          sK[kk][2 * j + 1] = c;
          sV[kk][2 * j] = v[off + 2 * j];
          sV[kk][2 * j + 1] = v[off + 2 * j + 1];
        }
        if (R > 0) {
          for (int t = ch; t < R; t += 4) sK[kk][D + t] = bv[((int64_t)h * N + key) * R + t];
        }
        if (ch == 0) sLab[kk] = axis_label(wy * M + kr, P.Hg, M, s) * 3 + axis_label(wx * M + kcc, P.Wg, M, s);
      }
    }
    __syncthreads();
    if (valid) {
      for (int kk = 0; kk < kc; ++kk) {
        if (sLab[kk] != qlab) continue;
        float sc = 0.f;
#pragma unroll
        for (int j = 0; j < D; ++j) sc = fmaf(qv[j], sK[kk][j], sc);
        if (R > 0) {
#pragma unroll
          for (int t = 0; t < R; ++t) sc = fmaf(uq[t], sK[kk][D + t], sc);
        }
        if (sc > m) {
          const float a = expf(m - sc);  // m = -inf on the first key gives 0
          l *= a;
#pragma unroll
          for (int j = 0; j < D; ++j) o[j] *= a;
          m = sc;
        }
        const float p = expf(sc - m);
        l += p;
#pragma unroll
        for (int j = 0; j < D; ++j) o[j] = fmaf(p, sV[kk][j], o[j]);
      }
    }
    __syncthreads();
  }
  if (valid) {
    float* dst = out + offset(qr, qc);
    const float inv = 1.0f / l;
#pragma unroll
    for (int j = 0; j < D; ++j) dst[j] = o[j] * inv;
  }
}

}  // namespace

// ------------------------------------------------------------------------------------
// Launchers (C++ linkage, internal to the library)
// ------------------------------------------------------------------------------------

template <int NKS, bool ROPE, bool OUTF32>
static void launch_bf16_inst(const WattnPlan& plan, const void* q, const void* k, const void* v, void* out,
                             const float* theta, const void* bu, const void* bv, hipStream_t stream) {
  hipLaunchKernelGGL((wattn_fwd_bf16_kernel<NKS, ROPE, OUTF32>), dim3(plan.grid), dim3(NTHR), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), out, theta, static_cast<const uint16_t*>(bu),
                     static_cast<const uint16_t*>(bv), plan);
}

hipError_t wattn_launch_bf16(const WattnPlan& plan, int nks, bool rope, bool out_f32, const void* q,
                             const void* k, const void* v, void* out, const float* theta, const void* bu,
                             const void* bv, hipStream_t stream) {
  const int sel = (nks == 3 ? 4 : 0) + (rope ? 2 : 0) + (out_f32 ? 1 : 0);
  switch (sel) {
    case 0: launch_bf16_inst<2, false, false>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 1: launch_bf16_inst<2, false, true>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 2: launch_bf16_inst<2, true, false>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 3: launch_bf16_inst<2, true, true>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 4: launch_bf16_inst<3, false, false>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 5: launch_bf16_inst<3, false, true>(plan, q, k, v, out, theta, bu, bv, stream); break;
    case 6: launch_bf16_inst<3, true, false>(plan, q, k, v, out, theta, bu, bv, stream); break;
    default: launch_bf16_inst<3, true, true>(plan, q, k, v, out, theta, bu, bv, stream); break;
  }
  return hipGetLastError();
}

hipError_t wattn_launch_f32(const WattnF32Plan& plan, int r, const void* q, const void* k, const void* v,
                            void* out, const float* theta, const void* bu, const void* bv, hipStream_t stream) {
  const dim3 grid(plan.grid), block(256);
  auto Q = static_cast<const float*>(q);
  auto K = static_cast<const float*>(k);
  auto V = static_cast<const float*>(v);
  auto O = static_cast<float*>(out);
  auto U = static_cast<const float*>(bu);
  auto W = static_cast<const float*>(bv);
  if (r == 16)
    hipLaunchKernelGGL((wattn_fwd_f32_kernel<16>), grid, block, 0, stream, Q, K, V, O, theta, U, W, plan);
  else
    hipLaunchKernelGGL((wattn_fwd_f32_kernel<0>), grid, block, 0, stream, Q, K, V, O, theta, U, W, plan);
  return hipGetLastError();
}
