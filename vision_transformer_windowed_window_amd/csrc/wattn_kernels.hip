// wattn_kernels.hip -- device code of libwattn.so for gfx950 (AMD Instinct MI355X).
//
// Fused shifted-window attention (FLASHSWIN page, "How it works", first and second
// changes; RIB page, section 2.1 for the bias channels).  One workgroup owns 256 queries
// of one wrap region of one window and head, and streams that region's keys through LDS
// in tiles of 64:
//
//   prologue : decode the task; build the window-local cos/sin table of the head in LDS
//              (angles in fp64, stored as fp32); load this wave's 64 queries straight from
//              their original (un-shifted) grid positions, rotate them in fp32, fold in
//              d^-1/2 * log2(e), round once to bf16 and keep them in registers; append the
//              bias channels u * log2(e) when the call has a bias.
//   key loop : per tile, every thread fetches one 16-byte chunk of K and of V (and of the
//              bias factor v) for the next tile while the current one is computed, then
//              rotates K in fp32, rounds it to bf16 and writes K and V^T into the other LDS
//              buffer.  Per 32-key step and 32-query block a wave runs
//                  S^T = K Q^T        on 32x32x16 bf16 MFMA, accumulator preset to -m,
//                  p   = 2^(S^T)      online softmax in fp32 registers,
//                  O^T += V^T P^T     on 32x32x16 bf16 MFMA.
//              Computing the transposed products keeps every query's scores, running
//              max m, running sum l and output accumulator in the same lane.
//   epilogue : O / l, stored as bf16 (rounded to nearest even) or as fp32, at the tokens'
//              original grid positions (this reverses the cyclic shift).
//
// The running max is updated lazily: the accumulator starts from -m, so S^T already holds
// s - m and p = 2^(s - m) costs one exp per score.  The exact rescale (row max, O and l
// scaled by 2^-(delta)) runs only for the first key step and whenever some p of a step
// exceeds 2^16, which bounds every p by 2^16 (no overflow: at most 2^16 * N per row sum).
// Row sums are taken over the bf16-rounded p that the PV product consumes.
//
// The fp32 path (wattn_fwd_f32_kernel) is a plain per-query loop over the whole window
// with the region-label mask, used for float32 inputs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wattn_plan.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 32;          // head dimension of q, k, v
constexpr int NTHR = 256;      // threads per workgroup (4 waves)
constexpr int QT = 256;        // queries per workgroup (64 per wave, 2 blocks of 32)
constexpr int KT = 64;         // keys per LDS tile
constexpr int VTS = KT + 8;    // row stride (elements) of the transposed V tile
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

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
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

// Swizzle of the four 16-byte chunks of a K row in LDS: the eight rows read together by
// one MFMA operand load fall into eight distinct bank groups.
__device__ __forceinline__ int kswz(int key) { return ((key >> 1) & 1) | (((key >> 4) & 1) << 1); }

// Row of the K tile that feeds MFMA A-operand row i (0..31): the accumulator row layout of
// the 32x32 MFMA then gives lane (query, g) the scores of keys 16g .. 16g+15 in order.
__device__ __forceinline__ int key_of_row(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

struct Task {
  int b, h, wy, wx, r0, rh, c0, rw, q0;
};

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
  t.wy = S.wy0 + wi / S.nwx;
  t.wx = S.wx0 + wi % S.nwx;
  t.r0 = S.r0;
  t.rh = S.rh;
  t.c0 = S.c0;
  t.rw = S.rw;
  t.q0 = qt * QT;
  return true;
}

// Element offset of (image b, rolled row Y, rolled col X, head h): the token's original
// position is ((Y + s) mod Hg, (X + s) mod Wg).
__device__ __forceinline__ int64_t token_offset(const WattnPlan& P, int b, int h, int Y, int X) {
  int y = Y + P.s;
  if (y >= P.Hg) y -= P.Hg;
  int x = X + P.s;
  if (x >= P.Wg) x -= P.Wg;
  return ((((int64_t)b * P.Hg + y) * P.Wg + x) * P.H + h) * D;
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
  __shared__ __align__(16) uint16_t sKb[BIAS ? 2 : 1][BIAS ? KT * 16 : 8];
  __shared__ __align__(16) uint16_t sVt[2][D * VTS];
  __shared__ float2 sTab[ROPE ? MAXM * (D / 2) : 1];

  Task T;
  if (!decode_task(P, blockIdx.x, T)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = P.M;
  const int h = T.h, b = T.b;
  const int n = T.rh * T.rw;
  const int wY = T.wy * M + T.r0, wX = T.wx * M + T.c0;  // rolled position of the region origin
  const Divider div(T.rw);

  if (ROPE) {
    for (int i = tid; i < M * (D / 2); i += NTHR) {
      const int pos = i >> 4, j = i & 15;
      double sn, cs;
      sincos((double)pos * (double)theta[h * (D / 2) + j], &sn, &cs);
      sTab[i] = make_float2((float)cs, (float)sn);
    }
    __syncthreads();
  }

  const int qi = lane & 31, g = lane >> 5;

  // ---- queries: rotate in fp32, scale by d^-1/2 * log2(e), round once to bf16
  u32x4 Qf[2][NKS];
  const float qscale = LOG2E * 0.17677669529663687f;  // log2(e) / sqrt(32)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int iq = T.q0 + wave * 64 + qb * 32 + qi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) Qf[qb][ks] = u32x4{0u, 0u, 0u, 0u};
    if (iq < n) {
      int lr, lc;
      div.split((uint32_t)iq, lr, lc);
      const int64_t off = token_offset(P, b, h, wY + lr, wX + lc);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(q + off + 16 * ks + 8 * g);
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float a = bf_lo(raw[p]), c = bf_hi(raw[p]);
          if (ROPE) {
            const int pos = (ks == 0) ? (T.r0 + lr) : (T.c0 + lc);
            const float2 t = sTab[pos * (D / 2) + 8 * ks + 4 * g + p];
            const float a2 = a * t.x - c * t.y;
            const float c2 = a * t.y + c * t.x;
            a = a2;
            c = c2;
          }
          o[p] = pack_bf16(a * qscale, c * qscale);
        }
        Qf[qb][ks] = o;
      }
      if (BIAS) {
        const int nl = (T.r0 + lr) * M + (T.c0 + lc);
        const u32x4 raw = *reinterpret_cast<const u32x4*>(bu + ((int64_t)h * M * M + nl) * 16 + 8 * g);
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = pack_bf16(bf_lo(raw[p]) * LOG2E, bf_hi(raw[p]) * LOG2E);
        Qf[qb][NKS - 1] = o;
      }
    }
  }
  const bool qb_live0 = T.q0 + wave * 64 < n;
  const bool qb_live1 = T.q0 + wave * 64 + 32 < n;

  // ---- loader state: K/V chunk (key lk of the tile, channels 8*lch .. 8*lch+7)
  const int lk = tid >> 2, lch = tid & 3;
  const int bk = tid >> 1, bch = tid & 1;  // bias-factor chunk (threads 0..127)
  u32x4 pk = {0u, 0u, 0u, 0u}, pv = {0u, 0u, 0u, 0u}, pb = {0u, 0u, 0u, 0u};
  int lpos = 0;

  auto fetch = [&](int tile) {
    const int key = tile * KT + lk;
    pk = u32x4{0u, 0u, 0u, 0u};
    pv = u32x4{0u, 0u, 0u, 0u};
    lpos = 0;
    if (key < n) {
      int lr, lc;
      div.split((uint32_t)key, lr, lc);
      const int64_t off = token_offset(P, b, h, wY + lr, wX + lc) + 8 * lch;
      pk = *reinterpret_cast<const u32x4*>(k + off);
      pv = *reinterpret_cast<const u32x4*>(v + off);
      lpos = (lch < 2) ? (T.r0 + lr) : (T.c0 + lc);
    }
    if (BIAS) {
      pb = u32x4{0u, 0u, 0u, 0u};
      const int key2 = tile * KT + bk;
      if (tid < 2 * KT && key2 < n) {
        int lr, lc;
        div.split((uint32_t)key2, lr, lc);
        const int nl = (T.r0 + lr) * M + (T.c0 + lc);
        pb = *reinterpret_cast<const u32x4*>(bv + ((int64_t)h * M * M + nl) * 16 + 8 * bch);
      }
    }
  };

  auto store = [&](int buf) {
    u32x4 kr = pk;
    if (ROPE) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = bf_lo(pk[p]), c = bf_hi(pk[p]);
        const float2 t = sTab[lpos * (D / 2) + 4 * lch + p];
        kr[p] = pack_bf16(a * t.x - c * t.y, a * t.y + c * t.x);
      }
    }
    *reinterpret_cast<u32x4*>(&sK[buf][lk * D + ((lch ^ kswz(lk)) * 8)]) = kr;
    uint16_t* vt = &sVt[buf][(8 * lch) * VTS + lk];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      vt[(2 * p) * VTS] = (uint16_t)(pv[p] & 0xffffu);
      vt[(2 * p + 1) * VTS] = (uint16_t)(pv[p] >> 16);
    }
    if (BIAS && tid < 2 * KT)
      *reinterpret_cast<u32x4*>(&sKb[buf][bk * 16 + ((bch ^ ((bk >> 4) & 1)) * 8)]) = pb;
  };

  // ---- per-query online-softmax state (lane = query; both halves g hold the same m)
  f32x16 O[2], Cn[2];
  float m[2], l[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m[qb] = 0.f;
    l[qb] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      O[qb][e] = 0.f;
      Cn[qb][e] = 0.f;
    }
  }
  const uint32_t ONES = 0x3f803f80u;  // bf16 pair (1.0, 1.0)
  const int ntile = (n + KT - 1) / KT;

  fetch(0);
  store(0);
  __syncthreads();

  for (int tile = 0; tile < ntile; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntile) fetch(tile + 1);

#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb = st * 32;
      const int kglob = tile * KT + kb;  // first key of the step
      if (kglob < n) {
        const int i = lane & 31;
        const int key = kb + key_of_row(i);
        u32x4 Kf[NKS];
        Kf[0] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + (((0 + g) ^ kswz(key)) * 8)]);
        Kf[1] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + (((2 + g) ^ kswz(key)) * 8)]);
        if (BIAS)
          Kf[NKS - 1] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 16 + ((g ^ ((key >> 4) & 1)) * 8)]);
        u32x4 Vf[2];
        Vf[0] = *reinterpret_cast<const u32x4*>(&sVt[buf][i * VTS + kb + 16 * g]);
        Vf[1] = *reinterpret_cast<const u32x4*>(&sVt[buf][i * VTS + kb + 16 * g + 8]);
        const bool partial = kglob + 32 > n;
        const bool first = (tile == 0) && (st == 0);

#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (!(qb == 0 ? qb_live0 : qb_live1)) continue;
          f32x16 S = mfma32(Kf[0], Qf[qb][0], Cn[qb]);
#pragma unroll
          for (int ks = 1; ks < NKS; ++ks) S = mfma32(Kf[ks], Qf[qb][ks], S);
          if (partial) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (kglob + 16 * g + e >= n) S[e] = -INFINITY;
          }
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
              l[qb] *= a;
#pragma unroll
              for (int e = 0; e < 16; ++e) O[qb][e] *= a;
            }
            m[qb] += delta;
#pragma unroll
            for (int e = 0; e < 16; ++e) Cn[qb][e] = -m[qb];
            ls = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              Pp[t] = pack_bf16(__builtin_amdgcn_exp2f(S[2 * t] - delta), __builtin_amdgcn_exp2f(S[2 * t + 1] - delta));
              ls = dot2_bf16(Pp[t], ONES, ls);
            }
          }
          l[qb] += ls;
          const u32x4 P0 = {Pp[0], Pp[1], Pp[2], Pp[3]};
          const u32x4 P1 = {Pp[4], Pp[5], Pp[6], Pp[7]};
          O[qb] = mfma32(Vf[0], P0, O[qb]);
          O[qb] = mfma32(Vf[1], P1, O[qb]);
        }
      }
    }

    if (tile + 1 < ntile) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round, scatter to the original positions
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int iq = T.q0 + wave * 64 + qb * 32 + qi;
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    if (iq < n) {
      const float inv = 1.0f / lt;
      int lr, lc;
      div.split((uint32_t)iq, lr, lc);
      const int64_t off = token_offset(P, b, h, wY + lr, wX + lc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (OUTF32) {
          const float4 w = make_float4(O[qb][4 * t + 0] * inv, O[qb][4 * t + 1] * inv, O[qb][4 * t + 2] * inv,
                                       O[qb][4 * t + 3] * inv);
          *reinterpret_cast<float4*>(static_cast<float*>(out) + off + 8 * t + 4 * g) = w;
        } else {
          u32x2 w;
          w[0] = pack_bf16(O[qb][4 * t + 0] * inv, O[qb][4 * t + 1] * inv);
          w[1] = pack_bf16(O[qb][4 * t + 2] * inv, O[qb][4 * t + 3] * inv);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + off + 8 * t + 4 * g) = w;
        }
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
