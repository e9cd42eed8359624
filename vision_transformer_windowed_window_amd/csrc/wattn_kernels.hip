// wattn_kernels.hip -- device code of libwattn.so for gfx950 (AMD Instinct MI355X).
//
// Fused shifted-window attention (FLASHSWIN page, "How it works", first and second
// changes; RIB page, section 2.1 for the bias channels).
//
// Work decomposition.  A shifted window of the last row or column band holds two (corner:
// four) wrap regions; tokens attend only within their region, and each region is a
// rectangle of tokens that is contiguous in the ORIGINAL (un-shifted) grid.  A workgroup
// of NW waves (2, 4 or 8, picked by the host from the window side) owns 32 NW queries (32
// per wave, two blocks of 16) of one region of one window and head and streams the
// region's keys through LDS in tiles of 16 NW keys.  The masked pairs of the shifted layer
// are never computed.
//
//   prologue : decode the task; issue the global loads of the head's angles, the wave's
//              queries and the first K/V tile together; build the window-local cos/sin
//              table in LDS (fp32 angles, hardware sin/cos); rotate the queries in fp32,
//              fold in d^-1/2 * log2(e), round once to fp16 and keep them in registers;
//              with a bias, u * log2(e) forms a second (zero-padded) k = 32 operand.
//   key loop : per tile, every thread fetches one 16-byte chunk of K and the matching
//              chunk of V (half the threads also one of the bias factor v) for the next tile
//              while the current tile is computed; then K is rotated in fp32, rounded to
//              fp16 and stored with V (bf16, unchanged) into the other LDS buffer (both
//              row-major, chunk-swizzled against bank conflicts).  Per 32-key step and
//              16-query block each wave runs
//                  S^T = K Q^T        16x16x32 fp16 MFMA (k = d = 32), accumulator preset
//                                     to -m, one product per 16 keys,
//                  p   = 2^(S^T)      fp32 online softmax in registers,
//                  O^T += V^T P^T     16x16x32 bf16 MFMA per 16 dims, V^T read with
//                                     ds_read_b64_tr_b16.
//              The transposed products keep each query's scores, running max m, running
//              sum l and output column in one lane column: lanes c, c+16, c+32, c+48 hold
//              query c of a block and split its keys (and output dims) four ways.
//   epilogue : O / l, stored as bf16 (round to nearest even) or fp32 at the tokens'
//              original positions, which reverses the cyclic shift.
//
// All chained products use the same MFMA instruction (16x16x32), so they complete in issue
// order: a shorter MFMA issued right after a longer one could otherwise write registers the
// longer one still reads as its accumulator input.
//
// The running max is updated lazily: with the accumulator preset to -m, S^T already holds
// s - m and p = 2^(s - m) costs one exp per score.  The exact rescale (row max, O and l
// scaled by 2^-delta) runs for the first key step and whenever the eight p a lane adds to
// its row sum in one step exceed 2^16 in total, so every p that reaches O stays within
// [0, 2^16] up to rounding (row sums stay below 2^16 * N).  Row sums are taken over the
// bf16-rounded p that the PV product consumes, chained into the running sum with dot2
// instructions; the step's share is the difference to the sum before the step.
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

#include <type_traits>

#include "wattn_plan.h"

namespace {

#include "wattn_device.h"

constexpr int MAXM = 128;      // largest window side (cos/sin table rows)

// 1 / (1 + e^-z) with the hardware exp2 and reciprocal (fp32, about 1 ulp each); z = -inf
// gives 0, z = +inf gives 1, NaN stays NaN.
__device__ __forceinline__ float sigmoidf_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * LOG2E));
}
constexpr float REF_HEADROOM = 16.0f;  // the forward reference sits this far (base 2) above the row maximum

struct Task {
  int b, h, q0;
  int qt, nqt;         // tile index within the region-head and its tile count (tasks qt - .. are consecutive)
  int r0, rh, c0, rw;  // region in window-local coordinates
  int y0, x0;          // region origin in the original grid (the region does not wrap)
  int step_i, step_j;  // one key tile as region rows and columns
  uint32_t rw_magic;   // multiplier of the index split by rw
};

// Workgroup -> task.  Groups of `chunk` consecutive tasks (query tiles of one region and
// head, which share K/V) go to one XCD (workgroups are dealt to the 8 XCDs round-robin), so
// their K/V lines meet in one L2.  The grid is a multiple of 8 * chunk.
// x / d and x % d for uniform 0 <= x < 2^31, 1 <= d, with r = recip(d) from the host: the
// multiply-high under-estimates the quotient by at most one.
__device__ __forceinline__ void udivmod(uint32_t x, uint32_t d, uint32_t r, uint32_t& q, uint32_t& m) {
  q = __umulhi(x, r);
  m = x - q * d;
  if (m >= d) {
    q += 1;
    m -= d;
  }
}

__device__ __forceinline__ int task_of_block(const WattnPlan& P, int bid) {
  const uint32_t C = (uint32_t)P.chunk;
  const uint32_t xcd = (uint32_t)bid & 7, slot = (uint32_t)bid >> 3;
  uint32_t grp, sub;
  udivmod(slot, C, P.chunk_r, grp, sub);
  return (int)((grp * 8 + xcd) * C + sub);
}

__device__ __forceinline__ bool decode_task(const WattnPlan& P, int task, int QT, Task& t) {
  if (task >= P.ntasks) return false;
  int si = 0;
#pragma unroll
  for (int i = 1; i < WATTN_MAX_SEG; ++i)
    if (i < P.nseg && task >= P.seg[i].task_begin) si = i;
  const WattnSeg& S = P.seg[si];  // read on demand (dynamic index), not kept live across tasks
  uint32_t u = (uint32_t)(task - S.task_begin), qt, h, wi, b, wr, wc;
  udivmod(u, (uint32_t)S.nqt, S.nqt_r, u, qt);
  udivmod(u, (uint32_t)P.H, P.H_r, u, h);
  udivmod(u, (uint32_t)(S.nwy * S.nwx), S.nwin_r, b, wi);
  udivmod(wi, (uint32_t)S.nwx, S.nwx_r, wr, wc);
  t.h = (int)h;
  t.b = (int)b;
  t.step_i = S.step_i;
  t.step_j = S.step_j;
  t.rw_magic = S.rw_magic;
  const int wy = S.wy0 + (int)wr;
  const int wx = S.wx0 + (int)wc;
  t.r0 = S.r0;
  t.rh = S.rh;
  t.c0 = S.c0;
  t.rw = S.rw;
  t.q0 = (int)qt * QT;
  t.qt = (int)qt;
  t.nqt = S.nqt;
  int y = wy * P.M + S.r0 + P.s;
  if (y >= P.Hg) y -= P.Hg;
  int x = wx * P.M + S.c0 + P.s;
  if (x >= P.Wg) x -= P.Wg;
  t.y0 = y;
  t.x0 = x;
  return true;
}

// Wave-uniform quantities of one task.
struct TaskCtx {
  Task t;
  int n;                 // tokens of the region
  int64_t img;           // element offset of the image
  int regbase;           // element offset (within the image) of the region origin, head h
  int ntile;             // key tiles
  int step_i, step_j;    // region coordinates advanced per tile
  int step_off;          // element offset advanced per tile without a column carry
  int carry_off;         // extra offset on a column carry
  uint32_t den, magic;   // division by the region width
};

__device__ __forceinline__ TaskCtx make_ctx(const WattnPlan& P, const Task& t, int KT) {
  TaskCtx X;
  X.t = t;
  X.n = t.rh * t.rw;
  const int colstride = P.H * D, rowstride = P.Wg * colstride;
  X.img = (int64_t)t.b * P.Hg * rowstride;
  X.regbase = t.y0 * rowstride + t.x0 * colstride + t.h * D;
  X.ntile = (X.n + KT - 1) / KT;
  X.step_i = t.step_i;
  X.step_j = t.step_j;
  X.step_off = X.step_i * rowstride + X.step_j * colstride;
  X.carry_off = rowstride - t.rw * colstride;
  X.den = (uint32_t)t.rw;
  X.magic = t.rw_magic;
  return X;
}

// i / den and i % den for 0 <= i < 2^16 (den <= 2^16), via a multiply-high.
__device__ __forceinline__ void split_idx(const TaskCtx& X, uint32_t i, int& qt, int& rm) {
  const uint32_t qq = (X.den == 1) ? i : __umulhi(i, X.magic);
  qt = (int)qq;
  rm = (int)(i - qq * X.den);
}

// Row stride (entries) of the cos/sin table for the window sides each width serves (up to 18, 26
// and 128); 32 * stride bytes is 64 mod 256, so the four chunks of a key read distinct banks.
__host__ __device__ constexpr int table_stride(int NW) { return NW == 2 ? 18 : (NW == 4 ? 26 : 130); }

// NW waves per workgroup (2, 4 or 8): 32 NW queries, key tiles of 16 NW keys.
// NKS: 16-channel groups of the score product's contraction: 2 (d = 32, no bias), 3 (a rank-16
// bias, zero-padded to a second k = 32 product) or 4 (a rank-32 bias, one full k = 32 product).
// Every form runs four waves per SIMD (at most 128 VGPRs) except the 8-wave rank-16 kernel,
// which needs more registers and runs one workgroup per CU.
template <int NW, int NKS, bool ROPE, bool OUTF32, bool GATE>
__global__ __launch_bounds__(64 * NW, (NKS == 3 && NW == 8) ? 2 : 4) void wattn_fwd_bf16_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              void* __restrict__ out,
                                                              const float* __restrict__ theta,
                                                              const uint16_t* __restrict__ bu,
                                                              const uint16_t* __restrict__ bv,
                                                              float* __restrict__ lse,
                                                              const uint16_t* __restrict__ gz,
                                                              const WattnPlan P) {
  constexpr bool BIAS = (NKS >= 3);
  constexpr int BR = (NKS - 2) * 16;          // bias channels (0, 16 or 32)
  constexpr int NTHR = 64 * NW;  // threads
  constexpr int QT = 32 * NW;    // queries (two 16-query blocks per wave)
  constexpr int KT = 16 * NW;    // keys per LDS tile: each thread stages one 16-byte chunk of K and of V
  __shared__ __align__(16) uint16_t sK[2][KT * D];
  __shared__ __align__(16) uint16_t sV[2][KT * D];
  __shared__ __align__(16) uint16_t sKb[BIAS ? 2 : 1][BIAS ? KT * BR : 8];
  constexpr int TSTR = table_stride(NW);
  extern __shared__ float2 sTab[];  // 16 rows of TSTR cos/sin entries of the head, pair-major (dynamic size)

  const int tid = threadIdx.x;
  Task T0;
  if (!decode_task(P, task_of_block(P, blockIdx.x), QT, T0)) return;
  const TaskCtx X = make_ctx(P, T0, KT);

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = P.M;
  const int colstride = P.H * D;            // elements between horizontally adjacent tokens
  const int rowstride = P.Wg * colstride;   // elements between vertically adjacent tokens

  // Lane (c, g): column c of every 16x16 MFMA block, k-group / row-group g.
  const int c = lane & 15, g = lane >> 4;
  const bool tab_thread = ROPE && tid < M * (D / 2);  // one table entry per thread

  // ---- per-task loads that are issued ahead of their use: the head's angle for this
  //      thread's table entry, and this lane's raw query chunks (bias: u chunks).
  float th = 0.f;
  u32x4 qraw[2];
  u32x4 braw[2];
  int qpos[2];
  auto load_task_inputs = [&](const TaskCtx& Y) {
    if (tab_thread) th = theta[Y.t.h * (D / 2) + (tid & 15)];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      qraw[a] = u32x4{0u, 0u, 0u, 0u};
      braw[a] = u32x4{0u, 0u, 0u, 0u};
      qpos[a] = 0;
      const int iq = Y.t.q0 + wave * 32 + 16 * a + c;
      if (iq < Y.n) {
        int li, lj;
        split_idx(Y, (uint32_t)iq, li, lj);
        const int off = Y.regbase + li * rowstride + lj * colstride;
        qraw[a] = *reinterpret_cast<const u32x4*>(q + Y.img + off + 8 * g);
        qpos[a] = (g < 2) ? (Y.t.r0 + li) : (Y.t.c0 + lj);  // channels 0..15 carry y, 16..31 x
        if (BIAS && 8 * g < BR) {
          const int nl = (Y.t.r0 + li) * M + (Y.t.c0 + lj);
          braw[a] = *reinterpret_cast<const u32x4*>(bu + ((int64_t)Y.t.h * M * M + nl) * BR + 8 * g);
        }
      }
    }
  };
  // window-local cos/sin table of the head (fp32 angles, hardware sin/cos)
  auto build_table = [&](const TaskCtx& Y) {
    if (ROPE) {
      if (tab_thread) {
        float sn, cs;
        __sincosf((float)(tid >> 4) * th, &sn, &cs);
        sTab[(tid & 15) * TSTR + (tid >> 4)] = make_float2(cs, sn);
      }
      for (int i = tid + NTHR; i < M * (D / 2); i += NTHR) {  // the entries beyond one per thread
        const int pos = i >> 4, j = i & 15;
        float sn, cs;
        __sincosf((float)pos * theta[Y.t.h * (D / 2) + j], &sn, &cs);
        sTab[j * TSTR + pos] = make_float2(cs, sn);
      }
    }
  };
  // queries (B operand of the score product): query block a holds queries q0 + 32 wave +
  // 16 a + c; this lane keeps channels 8g .. 8g+7, rotated in fp32, scaled by
  // d^-1/2 * log2(e) and rounded once to fp16.  Bias: a second k = 32 operand holding
  // u * log2(e) in channels 0..15 (lanes g = 0, 1) and zeros in channels 16..31.
  u32x4 Qf[2];
  u32x4 Qb[2];
  auto make_queries = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float qscale = LOG2E * 0.17677669529663687f;  // log2(e) / sqrt(32)
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float x0 = bf_lo(qraw[a][p]), x1 = bf_hi(qraw[a][p]);
        if (ROPE) {
          const float2 t = sTab[(4 * g + p) * TSTR + qpos[a]];
          const float r0 = x0 * t.x - x1 * t.y;
          const float r1 = x0 * t.y + x1 * t.x;
          x0 = r0;
          x1 = r1;
        }
        o[p] = pack_f16(x0 * qscale, x1 * qscale);
      }
      Qf[a] = o;
      Qb[a] = u32x4{0u, 0u, 0u, 0u};
      if (BIAS) {
#pragma unroll
        for (int p = 0; p < 4; ++p) Qb[a][p] = pack_f16(bf_lo(braw[a][p]) * LOG2E, bf_hi(braw[a][p]) * LOG2E);
      }
    }
  };

  // ---- loader: thread t owns the 16-byte chunk lch = t % 4 of key lk = t / 4 of a tile in
  //      both K and V (same element offset) and the quarter lch of the key's bias-factor row
  //      (8 bytes at rank 16, 16 bytes at rank 32).  The key index advances by KT per tile;
  //      region coordinates and the element offset are carried along.  Keys past the region
  //      end load the region's last key (bias: the window's first position) -- finite data
  //      whose scores are masked, so their probabilities are exactly 0.
  const int lk = tid >> 2, lch = tid & 3;
  int ci, cj, koff, klast;
  u32x4 pk, pv, pb = {0u, 0u, 0u, 0u};
  int lpos = 0;
  auto loader_init = [&](const TaskCtx& Y) {
    split_idx(Y, (uint32_t)lk, ci, cj);
    koff = Y.regbase + ci * rowstride + cj * colstride + 8 * lch;
    int li, lj;
    split_idx(Y, (uint32_t)(Y.n - 1), li, lj);
    klast = Y.regbase + li * rowstride + lj * colstride + 8 * lch;
  };
  auto advance = [&](const TaskCtx& Y) {
    ci += Y.step_i;
    cj += Y.step_j;
    koff += Y.step_off;
    if (cj >= Y.t.rw) {
      cj -= Y.t.rw;
      ci += 1;
      koff += Y.carry_off;
    }
  };
  auto fetch = [&](const TaskCtx& Y, int tile) {
    const bool valid = tile * KT + lk < Y.n;
    // a 32-bit byte offset from the image base (a scalar address): no 64-bit address arithmetic
    const uint32_t off = (uint32_t)(valid ? koff : klast) * 2u;
    pk = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(k + Y.img) + off);
    pv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(v + Y.img) + off);
    lpos = (lch < 2) ? (Y.t.r0 + ci) : (Y.t.c0 + cj);
    if (BIAS) {
      const int key = valid ? (Y.t.r0 + ci) * M + (Y.t.c0 + cj) : 0;
      const uint16_t* src = bv + ((int64_t)Y.t.h * M * M + key) * BR + (BR / 4) * lch;
      if (BR == 16) {
        const u32x2 h = *reinterpret_cast<const u32x2*>(src);
        pb = u32x4{h[0], h[1], 0u, 0u};
      } else {
        pb = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };
  auto store = [&](int buf) {
    u32x4 kr;
    if (ROPE) {
      const int lp = min(lpos, M - 1);  // keys past the region end: any in-table row
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf_lo(pk[p]), x1 = bf_hi(pk[p]);
        const float2 t = sTab[(4 * lch + p) * TSTR + lp];
        kr[p] = pack_f16(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
      }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) kr[p] = pack_f16(bf_lo(pk[p]), bf_hi(pk[p]));
    }
    *reinterpret_cast<u32x4*>(&sK[buf][lk * D + ((lch ^ kswz(lk)) * 8)]) = kr;
    *reinterpret_cast<u32x4*>(&sV[buf][lk * D + ((lch ^ vswz(lk)) * 8)]) = pv;
    if (BIAS && BR == 16) {  // 32-byte rows: quarter lch is half lch / 2 (swizzled), offset 4 (lch % 2)
      const u32x2 br = {pack_f16(bf_lo(pb[0]), bf_hi(pb[0])), pack_f16(bf_lo(pb[1]), bf_hi(pb[1]))};
      *reinterpret_cast<u32x2*>(&sKb[buf][lk * 16 + 8 * ((lch >> 1) ^ bswz(lk)) + 4 * (lch & 1)]) = br;
    }
    if (BIAS && BR == 32) {  // 64-byte rows: the row layout of K
      u32x4 br;
#pragma unroll
      for (int p = 0; p < 4; ++p) br[p] = pack_f16(bf_lo(pb[p]), bf_hi(pb[p]));
      *reinterpret_cast<u32x4*>(&sKb[buf][lk * 32 + 8 * (lch ^ kswz(lk))]) = br;
    }
  };

  // per-lane constants of the operand reads
  const int krow = 8 * (c >> 2) + (c & 3);  // K tile row (within a step) of A-operand row c, key block 0
  const int vrow = 8 * g + (c >> 2);        // V tile row (within a step) of the transposed read, half 0
  const int vch = (c & 3) >> 1, vsub = 4 * (c & 1);
  const uint32_t ONES = 0x3f803f80u;        // bf16 pair (1.0, 1.0)

  // ---- prologue: the global loads of the angle table, the queries and the first K/V tile
  //      are issued together, so their latencies overlap.
  load_task_inputs(X);
  loader_init(X);
  fetch(X, 0);
  build_table(X);
  if (ROPE) __syncthreads();
  make_queries();
  store(0);
  advance(X);
  __syncthreads();

  // ---- online-softmax state per query block a (lanes c, c+16, c+32, c+48 share a query)
  f32x4 O[2][2];  // [dim block][query block]: dims 16 db + 4 g + e of query 16 a + c
  f32x4 L[2];     // row sums: every entry of L[a] is the running sum of query 16 a + c
  f32x4 Cn[2];    // -r broadcast, the accumulator preset of the score product
  float r[2];     // reference of the query (base 2): p = 2^(s - r)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    O[0][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    O[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    L[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    Cn[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    r[a] = 0.f;
  }
  const int n = X.n;
  const bool wave_live = X.t.q0 + wave * 32 < n;  // wave-uniform
  // bf16 ones: the row-sum operand.  Made opaque to the compiler, so that it stays in four
  // registers instead of being rebuilt from the constant with two moves in every step.
  u32x4 ONES4 = {ONES, ONES, ONES, ONES};
  asm volatile("" : "+v"(ONES4));

  // LDS operand fragments of one 32-key step
  struct KFrags {
    u32x4 Kf[2];  // score operand A: key kb + 8(c/4) + 4b + c%4, channels 8g .. 8g+7 (fp16)
    u32x4 Kb[2];  // bias operand A: channels 8(g%2) .. 8(g%2)+7 of the same keys
  };
  auto load_kfrags = [&](int buf, int kb, KFrags& F) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int key = kb + krow + 4 * b;
      F.Kf[b] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + ((g ^ kswz(key)) * 8)]);
      if (BIAS && BR == 16) F.Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 16 + 8 * ((g & 1) ^ bswz(key))]);
      if (BIAS && BR == 32) F.Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 32 + 8 * (g ^ kswz(key))]);
    }
  };
  // value operand A (V^T): dims 16 db + c, keys kb + 8g .. 8g+7
  auto load_vfrags = [&](int buf, int kb, u32x4 (&Vf)[2]) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      u32x2 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = kb + vrow + 4 * hh;
        const int ch = 2 * db + vch;
        h[hh] = lds_read_tr16(&sV[buf][row * D + ((ch ^ vswz(row)) * 8) + vsub]);
      }
      Vf[db] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
    }
  };

  // One key tile: up to four 32-key steps.  Without a bias the score fragments of step st + 1
  // are read from LDS while step st is computed; the value fragments of a step are read at its
  // start and land while its exponentials run.
  //
  // Lazy reference: p = 2^(s - r) with r at least 16 above every score seen when it was
  // set, so p <= 2^-16 until a score exceeds the running maximum by more than 16.  A step
  // in which some p reaches 2 (bf16 exponent bit 7 set in one of the packed pairs; an
  // overflow to inf sets it too) is redone exactly: r grows to the step's row maximum + 16
  // and O and the row sums are scaled by 2^-delta.  Row sums are accumulated on the matrix
  // core (bf16 ones times P^T), over exactly the bf16 P the value product consumes.
  auto compute_tile = [&](int buf, int tile) {
    if (!wave_live) return;
    const int nst = min(KT / 32, (n - tile * KT + 31) / 32);  // steps holding keys (uniform)
    // Without a bias the score fragments of step st + 1 are read during step st (double
    // buffer).  With a bias they are read at the start of their own step: the 16 registers
    // saved bring the 4-wave kernel to 128 VGPRs, four waves per SIMD instead of three.
    constexpr bool KDB = !BIAS;
    KFrags F[KDB ? 2 : 1];
    load_kfrags(buf, 0, F[0]);
#pragma unroll
    for (int st = 0; st < KT / 32; ++st) {
      if (st < nst) {
        const int kg = tile * KT + st * 32;  // first key of the step (uniform)
        if (!KDB && st > 0) load_kfrags(buf, st * 32, F[0]);
        const KFrags& cur = F[KDB ? (st & 1) : 0];
        u32x4 Vf[2];
        load_vfrags(buf, st * 32, Vf);
        if (KDB && st + 1 < nst) load_kfrags(buf, (st + 1) * 32, F[(st + 1) & 1]);

        // S^T blocks: S[a][b][e] = score of query 16a + c and key kb + 8g + 4b + e, minus r
        f32x4 S[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            // bias channels first (the same k = 32 instruction as the score product, so
            // chained products complete in issue order)
            S[a][b] = BIAS ? mfma16_f16(cur.Kb[b], Qb[a], Cn[a]) : Cn[a];
            S[a][b] = mfma16_f16(cur.Kf[b], Qf[a], S[a][b]);
          }
        if (kg + 32 > n) {
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (kg + 8 * g + 4 * b + e >= n) S[a][b][e] = -INFINITY;
        }
        const bool first = (tile == 0) && (st == 0);
        uint32_t Pp[2][4];
        bool exact = first;
        if (!first) {
          uint32_t bits = 0u;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const f32x4& s = S[a][t >> 1];
              const int e0 = 2 * (t & 1);
              Pp[a][t] = pack_bf16(__builtin_amdgcn_exp2f(s[e0]), __builtin_amdgcn_exp2f(s[e0 + 1]));
              bits |= Pp[a][t];
            }
          exact = __any((bits & 0x40004000u) != 0u);  // some p >= 2 (or inf / NaN)
        }
        if (exact) {
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            float mx = fmaxf(fmaxf(S[a][0][0], S[a][0][1]), fmaxf(S[a][0][2], S[a][0][3]));
            mx = fmaxf(mx, fmaxf(fmaxf(S[a][1][0], S[a][1][1]), fmaxf(S[a][1][2], S[a][1][3])));
            mx = xmax32(xmax16(mx));
            // first step: reference = row max + 16; later: grow only where the step passed r
            const float delta = (first || mx > 0.f) ? mx + REF_HEADROOM : 0.f;
            if (!first) {
              const float f = __builtin_amdgcn_exp2f(-delta);
              L[a] *= f;
              O[0][a] *= f;
              O[1][a] *= f;
            }
            r[a] += delta;
            Cn[a] = f32x4{-r[a], -r[a], -r[a], -r[a]};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const f32x4& s = S[a][t >> 1];
              const int e0 = 2 * (t & 1);
              Pp[a][t] = pack_bf16(__builtin_amdgcn_exp2f(s[e0] - delta), __builtin_amdgcn_exp2f(s[e0 + 1] - delta));
            }
          }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const u32x4 Pa = {Pp[a][0], Pp[a][1], Pp[a][2], Pp[a][3]};  // keys kb + 8g .. 8g+7 of query 16a + c
#pragma unroll
          for (int db = 0; db < 2; ++db) O[db][a] = mfma16_bf16(Vf[db], Pa, O[db][a]);
          L[a] = mfma16_bf16(ONES4, Pa, L[a]);
        }
      }
    }
  };


  for (int tile = 0; tile < X.ntile; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < X.ntile;
    if (more) fetch(X, tile + 1);
    compute_tile(buf, tile);
    if (more) {
      store(buf ^ 1);
      advance(X);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, scatter to the original positions
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const float lt = L[a][0];
    const int iq = X.t.q0 + wave * 32 + 16 * a + c;
    if (iq < n) {
      const float inv = 1.0f / lt;
      int li, lj;
      split_idx(X, (uint32_t)iq, li, lj);
      const int64_t off = X.img + X.regbase + li * rowstride + lj * colstride;
      // natural-log log-sum-exp of the row: m and l are kept in base 2 (log2(e) folded into q)
      if (lse != nullptr && g == 0) lse[off / D] = (r[a] + __log2f(lt)) * LN2;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        f32x4 o = O[db][a] * inv;
        if (GATE) {  // out = sigmoid(z) * attention, z in q's type at the output position
          const u32x2 zr = *reinterpret_cast<const u32x2*>(gz + off + 16 * db + 4 * g);
          const float z[4] = {bf_lo(zr[0]), bf_hi(zr[0]), bf_lo(zr[1]), bf_hi(zr[1])};
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] *= sigmoidf_fast(z[e]);
        }
        if (OUTF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + off + 16 * db + 4 * g) =
              make_float4(o[0], o[1], o[2], o[3]);
        } else {
          const u32x2 wv = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + off + 16 * db + 4 * g) = wv;
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


// ------------------------------------------------------------------------------------
// Backward pass (flash-attention style: the scores are recomputed from the row log-sum-exp
// of the forward pass, never stored).  For one window, head and region, with natural-log
// logits s = (R q)(R k)^T / sqrt(d), P = exp(s - lse) and the output gradient dO:
//   D  = rowsum(dO * O),  dP = dO V^T,  dS = P * (dP - D),
//   dV = P^T dO,  d(Rq) = dS (Rk) / sqrt(d),  d(Rk) = dS^T (Rq) / sqrt(d),
//   dq = R^T d(Rq),  dk = R^T d(Rk),
//   dtheta[j] = sum over q and k tokens of pos_j * (g . J x) on rotation pair j, with g the
//   gradient and x the input of the token (a rotation and the quarter turn J commute).
// Kernel A owns query tiles and streams the region's K/V tiles (as the forward pass does):
// it writes D, dq and the q part of dtheta.  Kernel B owns key tiles and streams the
// region's rotated queries, dO and the per-query statistics: it writes dk, dv and the k
// part of dtheta.  Both use the same 16x16x32 MFMAs and LDS layouts as the forward pass.
// ------------------------------------------------------------------------------------

// Row stride (entries) of the backward kernels' cos/sin table for window side M: the
// smallest stride >= M that is 2 mod 8, so that 32 * stride bytes is 64 mod 256 and the four
// chunks of a row read distinct banks.  Sizing the table for the launch's own window (4.4 KB
// at M = 32 rather than 16.6 KB for the largest window) lets the query-tile kernel keep four
// workgroups on a CU.
__host__ __device__ constexpr int bwd_table_stride(int M) { return M + ((2 - M) & 7); }

// Region walk of one thread's row of a tile: region coordinates (ci, cj) and the element
// offset of key / query idx + tile * KT, advanced by one tile at a time.
struct Walker {
  int ci, cj, off, last;
};

__device__ __forceinline__ void walker_init(Walker& w, const TaskCtx& Y, int idx, int col, int rowstride,
                                            int colstride) {
  split_idx(Y, (uint32_t)idx, w.ci, w.cj);
  w.off = Y.regbase + w.ci * rowstride + w.cj * colstride + col;
  int li, lj;
  split_idx(Y, (uint32_t)(Y.n - 1), li, lj);
  w.last = Y.regbase + li * rowstride + lj * colstride + col;
}

__device__ __forceinline__ void walker_advance(Walker& w, const TaskCtx& Y) {
  w.ci += Y.step_i;
  w.cj += Y.step_j;
  w.off += Y.step_off;
  if (w.cj >= Y.t.rw) {
    w.cj -= Y.t.rw;
    w.ci += 1;
    w.off += Y.carry_off;
  }
}

// window-local cos/sin table (pair-major rows of TSTR entries), fp32 angles.  Every entry a
// thread writes belongs to pair tid % 16 (NTHR is a multiple of 16), so the caller loads that
// one angle, th, with its first batch of global loads.
template <int NTHR>
__device__ __forceinline__ void build_rope_table(float2* sTab, int TSTR, float th, int M, int tid) {
  static_assert(NTHR % 16 == 0, "one rotation pair per thread");
  for (int i = tid; i < M * (D / 2); i += NTHR) {
    float sn, cs;
    __sincosf((float)(i >> 4) * th, &sn, &cs);
    sTab[(i & 15) * TSTR + (i >> 4)] = make_float2(cs, sn);
  }
}

// eight bf16 or fp32 values of a gradient-side tensor (out or dout) as fp32
template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float x[8]) {
  if (F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      x[2 * p] = bf_lo(w[p]);
      x[2 * p + 1] = bf_hi(w[p]);
    }
  }
}

// un-rotate the gradient of four channels 4t' .. 4t'+3 (two rotation pairs j0, j0 + 1) at a
// window position and add the pairs' angle-gradient terms pos * (g . J x) to dth[0], dth[1]
template <bool ROPE>
__device__ __forceinline__ void finish_grad4(const f32x4 acc, float scale, int j0, int pos, const float2* sTab,
                                             int TSTR, const u32x2 raw, float dth[2], float out[4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float a = acc[2 * t] * scale, b = acc[2 * t + 1] * scale;
    if (ROPE) {
      const float2 cs = sTab[(j0 + t) * TSTR + pos];
      out[2 * t] = a * cs.x + b * cs.y;       // R^T: rotate back by -phi
      out[2 * t + 1] = -a * cs.y + b * cs.x;
    } else {
      out[2 * t] = a;
      out[2 * t + 1] = b;
    }
  }
  if (ROPE) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float x0 = bf_lo(raw[t]), x1 = bf_hi(raw[t]);
      dth[t] += (float)pos * (out[2 * t + 1] * x0 - out[2 * t] * x1);
    }
  }
}

// The angle gradient: each lane holds the terms of pairs 8 cb + 2 g + t (cb, t in {0, 1}) of its
// rows.  They are summed over the 16 lanes of a row group (DPP row, no LDS round trip), and each
// wave adds its 16 sums into copy (workgroup * NW + wave) % WATTN_DTHETA_COPIES of the head's
// partial sums, so that tens of thousands of waves do not queue on the same 16 addresses and no
// wave waits for the others of its workgroup; wattn_dtheta_reduce_kernel adds the copies up.
__device__ __forceinline__ float rowsum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror 4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror 8
  return x;
}
template <int NW>
__device__ __forceinline__ void dtheta_flush(float (&acc)[2][2], float* __restrict__ dth_part, int h, int H,
                                             int tid) {
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  // unsigned: the copy index stays in range for any grid size
  const uint32_t copy = ((uint32_t)blockIdx.x * NW + (uint32_t)(tid >> 6)) % WATTN_DTHETA_COPIES;
  float* dst = dth_part + ((int64_t)copy * H + h) * (D / 2);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float v = rowsum16(acc[cb][t]);
      if (c == 0) atomicAdd(dst + 8 * cb + 2 * g + t, v);
    }
}

// dS = P (dP - D) is rounded to fp16 for the products of dq and dk: its size follows dout,
// and training gradients are often small enough that dS would fall into fp16's subnormal
// range or to zero.  Both kernels therefore round 2^e dS instead, with e chosen from the
// largest output-gradient entry g_max so that 2^e g_max lies in [4, 8), and divide the
// accumulated products by 2^e in fp32.  The factor is folded into the score preset (P
// becomes 2^e P), so it costs no instruction per score.  The query-tile kernel takes e per
// query row (its products sum over keys only) and leaves the largest entry of its tile in
// one float per task; the key-tile kernel sums over the queries of its wrap region, so it
// takes one e per region from the largest of the region's tile entries (the tasks of a
// region and head are consecutive).
constexpr int GRAD_EXP_LIMIT = 96;
__device__ __forceinline__ int grad_scale_exp(float gmax) {
  const int e = 3 - __builtin_amdgcn_frexp_expf(gmax);  // gmax in [2^(x-1), 2^x): 2^e gmax in [4, 8)
  return max(-GRAD_EXP_LIMIT, min(GRAD_EXP_LIMIT, e));    // 0 and non-finite gmax give e = 3
}

// ---- Kernel A: dq (and D) per query tile; K/V streamed like the forward pass.  BR is the
//      bias rank (0, 16 or 32): the bias factors enter the scores as BR extra channels.
template <int NW, bool ROPE, bool OUTF32, int BR, bool GATE>
__global__ __launch_bounds__(64 * NW, BR ? 2 : 4) void wattn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ out, const void* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ delta, float* __restrict__ dq, float* __restrict__ dth_part, const float* __restrict__ theta,
    const uint16_t* __restrict__ bu, const uint16_t* __restrict__ bv, float* __restrict__ dbu,
    const uint16_t* __restrict__ gz, float* __restrict__ dz, uint16_t* __restrict__ qt,
    uint16_t* __restrict__ dot, float* __restrict__ tmax, const WattnPlan P) {
  constexpr int NTHR = 64 * NW, QT = 32 * NW, KT = 16 * NW;
  constexpr bool BIAS = BR > 0;
  constexpr int NBB = BR == 32 ? 2 : 1;  // 16-channel blocks of the bias gradient
  static_assert(BR == 0 || BR == 16 || BR == 32, "bias rank 0, 16 or 32");
  __shared__ __align__(16) uint16_t sK[2][KT * D];
  __shared__ __align__(16) uint16_t sV[2][KT * D];
  __shared__ __align__(16) uint16_t sKb[BIAS ? 2 : 1][BIAS ? KT * BR : 8];  // bias factor v of the keys (fp16)
  // the tile's raw q rows, for the dtheta terms of the epilogue (written and read by the same wave)
  __shared__ __align__(16) uint16_t sQraw[ROPE ? QT * D : 8];
  __shared__ float sGmax[NW];
  extern __shared__ float2 sTab[];

  const int tid = threadIdx.x;
  Task T0;
  const int task = task_of_block(P, blockIdx.x);
  if (!decode_task(P, task, QT, T0)) return;
  const TaskCtx X = make_ctx(P, T0, KT);
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int M = P.M, n = X.n;
  const int TSTR = bwd_table_stride(M);  // cos/sin table row stride
  const float th_tab = ROPE ? theta[X.t.h * (D / 2) + (tid & 15)] : 0.f;  // the angle of this thread's table entries
  const int colstride = P.H * D, rowstride = P.Wg * colstride;

  // ---- this lane's queries: q (rotated, scaled, fp16), dO (bf16), D and the row statistic
  //      (preset with the row's gradient-scale exponent); with a bias, u * log2(e) as a k = 32
  //      operand (rank 16: channels 0..15, zero-padded; rank 32: all of it)
  u32x4 qraw[2], dOf[2], Qb[2];
  f32x4 CnL[2], CnD[2];
  int qpos_r[2], qpos_c[2];
  int64_t qoff[2];
  bool qvalid[2];
  // all loads of both query blocks first, with no branch around them (a padded query's offset
  // is the region's first token, so every address is valid), so that they are in flight together
  float go[2][8], o[2][8], lraw[2];
  u32x4 zraw[2], braw[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int iq = X.t.q0 + wave * 32 + 16 * a + c;
    qvalid[a] = iq < n;
    int li = 0, lj = 0;
    if (qvalid[a]) split_idx(X, (uint32_t)iq, li, lj);
    qpos_r[a] = X.t.r0 + li;
    qpos_c[a] = X.t.c0 + lj;
    qoff[a] = X.img + X.regbase + li * rowstride + lj * colstride;
    qraw[a] = *reinterpret_cast<const u32x4*>(q + qoff[a] + 8 * g);
    load8<OUTF32>(dout, qoff[a] + 8 * g, go[a]);
    load8<OUTF32>(out, qoff[a] + 8 * g, o[a]);
    lraw[a] = lse[qoff[a] / D];
    if (GATE) zraw[a] = *reinterpret_cast<const u32x4*>(gz + qoff[a] + 8 * g);
    // rank 16: lanes g = 2, 3 reload the first half of the 16 bias channels and ignore it
    if (BIAS)
      braw[a] = *reinterpret_cast<const u32x4*>(
          bu + ((int64_t)X.t.h * M * M + qpos_r[a] * M + qpos_c[a]) * BR + 8 * (BR == 32 ? g : (g & 1)));
  }
  int gexp[2];     // gradient-scale exponent of each query row
  float wgmax = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float Dp = 0.f, L2 = 0.f;
    if (qvalid[a]) {
      L2 = lraw[a] * LOG2E;
      if (GATE) {
        // out is sigmoid(z) * attention: the attention's output gradient is dout * sigmoid(z),
        // dz = dout * out * (1 - sigmoid(z)), and D = rowsum(dout * out) is unchanged
#pragma unroll
        for (int e = 0; e < 8; ++e) Dp += go[a][e] * o[a][e];
        float gzv[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float s0 = sigmoidf_fast(bf_lo(zraw[a][p])), s1 = sigmoidf_fast(bf_hi(zraw[a][p]));
          gzv[2 * p] = go[a][2 * p] * o[a][2 * p] * (1.0f - s0);
          gzv[2 * p + 1] = go[a][2 * p + 1] * o[a][2 * p + 1] * (1.0f - s1);
          go[a][2 * p] *= s0;
          go[a][2 * p + 1] *= s1;
        }
        float* dst = dz + qoff[a] + 8 * g;
        *reinterpret_cast<float4*>(dst) = make_float4(gzv[0], gzv[1], gzv[2], gzv[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(gzv[4], gzv[5], gzv[6], gzv[7]);
      }
    } else {
      qraw[a] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) go[a][e] = 0.f;
    }
    if (ROPE) *reinterpret_cast<u32x4*>(&sQraw[(wave * 32 + 16 * a + c) * D + 8 * g]) = qraw[a];
#pragma unroll
    for (int p = 0; p < 4; ++p) dOf[a][p] = pack_bf16(go[a][2 * p], go[a][2 * p + 1]);
    // D from the same bf16 dO that dP uses, so that the row's dS = P (dP - D) sums to zero up
    // to the rounding of P, as it does exactly (with a gate: the given dout and out)
    if (!GATE && qvalid[a]) {
#pragma unroll
      for (int p = 0; p < 4; ++p) Dp += bf_lo(dOf[a][p]) * o[a][2 * p] + bf_hi(dOf[a][p]) * o[a][2 * p + 1];
    }
    const float Dn = xsum32(xsum16(Dp));  // the four lanes of query c hold 8 dims each
    if (qvalid[a] && g == 0) delta[qoff[a] / D] = Dn;
    float gm = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) gm = fmaxf(gm, fabsf(go[a][e]));
    gm = xmax32(xmax16(gm));  // largest entry of the row's (gated) output gradient
    wgmax = fmaxf(wgmax, gm);
    gexp[a] = grad_scale_exp(gm);
    L2 -= (float)gexp[a];     // P becomes 2^e P
    Qb[a] = u32x4{0u, 0u, 0u, 0u};
    if (BIAS && qvalid[a] && (BR == 32 || g < 2)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) Qb[a][p] = pack_f16(bf_lo(braw[a][p]) * LOG2E, bf_hi(braw[a][p]) * LOG2E);
    }
    CnL[a] = f32x4{-L2, -L2, -L2, -L2};
    CnD[a] = f32x4{-Dn, -Dn, -Dn, -Dn};
  }

  // ---- K/V tile loader (thread t: chunk t % 4 of key t / 4, in K and V; with a rank-32 bias
  //      the same chunk of the key's bias factor v; with rank 16, threads 0 .. 2 KT - 1 the
  //      16-byte half t % 2 of the bias factor v of key t / 2)
  const int lk = tid >> 2, lch = tid & 3;
  const int bk = BR == 32 ? lk : (tid % (2 * KT)) >> 1, bch = BR == 32 ? lch : tid & 1;
  const bool bthread = BIAS && (BR == 32 || tid < 2 * KT);
  Walker W, Wb;
  walker_init(W, X, lk, 8 * lch, rowstride, colstride);
  walker_init(Wb, X, bk, 0, rowstride, colstride);
  u32x4 pk, pv, pb = {0u, 0u, 0u, 0u};
  int lpos = 0;
  auto fetch = [&](int tile) {
    const bool valid = tile * KT + lk < n;
    const uint32_t off = (uint32_t)(valid ? W.off : W.last) * 2u;
    pk = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(k + X.img) + off);
    pv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(v + X.img) + off);
    lpos = (lch < 2) ? (X.t.r0 + W.ci) : (X.t.c0 + W.cj);
    if (bthread) {
      const int key = (tile * KT + bk < n) ? (X.t.r0 + Wb.ci) * M + (X.t.c0 + Wb.cj) : 0;
      pb = *reinterpret_cast<const u32x4*>(bv + ((int64_t)X.t.h * M * M + key) * BR + 8 * bch);
    }
  };
  auto store = [&](int buf) {
    u32x4 kr;
    const int lp = min(lpos, M - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = bf_lo(pk[p]), x1 = bf_hi(pk[p]);
      if (ROPE) {
        const float2 t = sTab[(4 * lch + p) * TSTR + lp];
        kr[p] = pack_f16(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
      } else {
        kr[p] = pack_f16(x0, x1);
      }
    }
    *reinterpret_cast<u32x4*>(&sK[buf][lk * D + ((lch ^ kswz(lk)) * 8)]) = kr;
    *reinterpret_cast<u32x4*>(&sV[buf][lk * D + ((lch ^ vswz(lk)) * 8)]) = pv;
    if (bthread) {
      u32x4 br;
#pragma unroll
      for (int p = 0; p < 4; ++p) br[p] = pack_f16(bf_lo(pb[p]), bf_hi(pb[p]));
      if (BR == 32)  // rows of 32 channels swizzled like K
        *reinterpret_cast<u32x4*>(&sKb[buf][bk * 32 + 8 * (bch ^ kswz(bk))]) = br;
      else
        *reinterpret_cast<u32x4*>(&sKb[buf][bk * 16 + 8 * (bch ^ bswz(bk))]) = br;
    }
  };

  // largest output-gradient entry of the tile, for the key-tile kernel's scale
  {
    float wm = wgmax;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) wm = fmaxf(wm, __shfl_xor(wm, o));  // lanes c of a row group
    if (lane == 0) sGmax[wave] = wm;                                      // xmax32/16 covered g
  }
  fetch(0);
  if (ROPE) build_rope_table<NTHR>(sTab, TSTR, th_tab, M, tid);
  __syncthreads();
  if (tid == 0) {
    float wm = sGmax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) wm = fmaxf(wm, sGmax[w]);
    tmax[task] = wm;  // every task of the launch writes its own slot
  }
  // queries: rotate (fp32), scale by log2(e) / sqrt(d), round to fp16
  u32x4 Qf[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const float qscale = LOG2E * 0.17677669529663687f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float x0 = bf_lo(qraw[a][p]), x1 = bf_hi(qraw[a][p]);
      if (ROPE) {
        const int j = 4 * g + p;
        const float2 t = sTab[j * TSTR + (j < D / 4 ? qpos_r[a] : qpos_c[a])];
        const float r0 = x0 * t.x - x1 * t.y, r1 = x0 * t.y + x1 * t.x;
        x0 = r0;
        x1 = r1;
      }
      Qf[a][p] = pack_f16(x0 * qscale, x1 * qscale);
    }
    // the key-tile kernel streams these operand-ready forms instead of re-deriving them
    if (qvalid[a]) {
      *reinterpret_cast<u32x4*>(qt + qoff[a] + 8 * g) = Qf[a];
      *reinterpret_cast<u32x4*>(dot + qoff[a] + 8 * g) = dOf[a];
    }
  }
  store(0);
  walker_advance(W, X);
  walker_advance(Wb, X);
  __syncthreads();

  const int krow = 8 * (c >> 2) + (c & 3);
  const int vrow = 8 * g + (c >> 2);
  const int vch = (c & 3) >> 1, vsub = 4 * (c & 1);
  f32x4 dQ[2][2];    // [channel block][query block]: channels 16 cb + 4 g + e of query 16 a + c
  f32x4 dU[NBB][2];  // [bias channel block][query block]: bias channels 16 cb + 4 g + e of query 16 a + c
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    dQ[0][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    dQ[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < NBB; ++cb) dU[cb][a] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bool wave_live = X.t.q0 + wave * 32 < n;

  for (int tile = 0; tile < X.ntile; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < X.ntile;
    if (more) fetch(tile + 1);
    if (wave_live) {
      // one 32-key block; MASK: the region's last, partial block, whose padded keys get -inf
      auto kblock = [&](int kb, int kg, auto mask_tag) {
          constexpr bool MASK = decltype(mask_tag)::value;
          u32x4 Kf[2], Vr[2], KTf[2], Kb[2], VbT[NBB];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int key = kb + krow + 4 * b;
            Kf[b] = *reinterpret_cast<const u32x4*>(&sK[buf][key * D + ((g ^ kswz(key)) * 8)]);
            Vr[b] = *reinterpret_cast<const u32x4*>(&sV[buf][key * D + ((g ^ vswz(key)) * 8)]);
            if (BR == 16) Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 16 + 8 * ((g & 1) ^ bswz(key))]);
            if (BR == 32) Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[buf][key * 32 + 8 * (g ^ kswz(key))]);
          }
          if (BIAS) {  // bias factor v^T: channel 16 cb + c, keys kb + 8 g .. 8 g + 7
#pragma unroll
            for (int cb = 0; cb < NBB; ++cb) {
              u32x2 h[2];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const int row = kb + vrow + 4 * hh;
                h[hh] = BR == 32 ? lds_read_tr16(&sKb[buf][row * 32 + (((2 * cb + vch) ^ kswz(row)) * 8) + vsub])
                                 : lds_read_tr16(&sKb[buf][row * 16 + ((vch ^ bswz(row)) * 8) + vsub]);
              }
              VbT[cb] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
            }
          }
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            u32x2 h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int row = kb + vrow + 4 * hh;
              h[hh] = lds_read_tr16(&sK[buf][row * D + (((2 * cb + vch) ^ kswz(row)) * 8) + vsub]);
            }
            KTf[cb] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
          }
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            f32x4 S[2], G[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              // log2-domain score minus the row statistic (bias channels first, as in the forward pass)
              S[b] = BIAS ? mfma16_f16(Kb[b], Qb[a], CnL[a]) : CnL[a];
              S[b] = mfma16_f16(Kf[b], Qf[a], S[b]);
              G[b] = mfma16_bf16(Vr[b], dOf[a], CnD[a]);  // dP - D
            }
            uint32_t dS16[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int b = t >> 1, e0 = 2 * (t & 1);
              float s0 = S[b][e0], s1 = S[b][e0 + 1];
              if (MASK) {
                if (kg + 8 * g + 4 * b + e0 >= n) s0 = -INFINITY;
                if (kg + 8 * g + 4 * b + e0 + 1 >= n) s1 = -INFINITY;
              }
              dS16[t] = pack_f16(__builtin_amdgcn_exp2f(s0) * G[b][e0], __builtin_amdgcn_exp2f(s1) * G[b][e0 + 1]);
            }
            const u32x4 dSa = {dS16[0], dS16[1], dS16[2], dS16[3]};
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) dQ[cb][a] = mfma16_f16(KTf[cb], dSa, dQ[cb][a]);
#pragma unroll
            for (int cb = 0; cb < NBB; ++cb)
              if (BIAS) dU[cb][a] = mfma16_f16(VbT[cb], dSa, dU[cb][a]);
          }
      };
#pragma unroll
      for (int st = 0; st < KT / 32; ++st) {
        const int kb = st * 32, kg = tile * KT + kb;
        if (kg + 32 <= n)
          kblock(kb, kg, std::false_type{});
        else if (kg < n)
          kblock(kb, kg, std::true_type{});
      }
    }
    if (more) {
      store(buf ^ 1);
      walker_advance(W, X);
      walker_advance(Wb, X);
    }
    __syncthreads();
  }

  // the query rows' addresses and window positions again: recomputed from an opaque copy of
  // the lane index, so that they are not held in registers across the key loop
  {
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int ce = lane_e & 15;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int iq = X.t.q0 + wave * 32 + 16 * a + ce;
      qvalid[a] = iq < n;
      int li = 0, lj = 0;
      if (qvalid[a]) split_idx(X, (uint32_t)iq, li, lj);
      qpos_r[a] = X.t.r0 + li;
      qpos_c[a] = X.t.c0 + lj;
      qoff[a] = X.img + X.regbase + li * rowstride + lj * colstride;
    }
  }
  // ---- epilogue: the gradient of the bias factor u (shared by every window and image: added
  //      into its window position with atomics), dq = R^T (dS K) / sqrt(d), the q part of dtheta
  if (BIAS) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (!qvalid[a]) continue;
      float* dst = dbu + ((int64_t)X.t.h * M * M + qpos_r[a] * M + qpos_c[a]) * BR + 4 * g;
      const float us = __builtin_ldexpf(1.0f, -gexp[a]);
#pragma unroll
      for (int cb = 0; cb < NBB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(dst + 16 * cb + e, dU[cb][a][e] * us);
    }
  }
  // the raw q channels of the dtheta sums (the prologue left the rows in LDS)
  u32x2 qr2[2][2] = {};
  if (ROPE) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        qr2[a][cb] = *reinterpret_cast<const u32x2*>(&sQraw[(wave * 32 + 16 * a + c) * D + 16 * cb + 4 * g]);
  }
  float dth[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // [channel block][pair]: this lane's angle-gradient terms
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (!qvalid[a]) continue;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float r4[4];
      const int pos = cb == 0 ? qpos_r[a] : qpos_c[a];  // channels 0..15 rotate with the row
      finish_grad4<ROPE>(dQ[cb][a], __builtin_ldexpf(0.17677669529663687f, -gexp[a]), 8 * cb + 2 * g, pos, sTab,
                         TSTR, qr2[a][cb], dth[cb], r4);
      *reinterpret_cast<float4*>(dq + qoff[a] + 16 * cb + 4 * g) = make_float4(r4[0], r4[1], r4[2], r4[3]);
    }
  }
  if (ROPE) dtheta_flush<NW>(dth, dth_part, X.t.h, P.H, tid);
}

// ---- Kernel B: dk, dv per key tile; rotated queries, dO and the per-query statistics streamed.
template <int NW, bool ROPE, int BR>
__global__ __launch_bounds__(64 * NW, 2) void wattn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ qt, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dot, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dth_part, const float* __restrict__ theta,
    const uint16_t* __restrict__ bu, const uint16_t* __restrict__ bv, float* __restrict__ dbv,
    const float* __restrict__ tmax, const WattnPlan P) {
  constexpr int NTHR = 64 * NW, KTW = 32 * NW, QTT = 16 * NW;  // keys per task, queries per tile
  constexpr bool BIAS = BR > 0;
  constexpr int NBB = BR == 32 ? 2 : 1;  // 16-channel blocks of the bias gradient
  static_assert(BR == 0 || BR == 16 || BR == 32, "bias rank 0, 16 or 32");
  __shared__ __align__(16) uint16_t sQ[2][QTT * D];
  __shared__ __align__(16) uint16_t sO[2][QTT * D];
  __shared__ __align__(16) uint16_t sUb[BIAS ? 2 : 1][BIAS ? QTT * BR : 8];  // u * log2(e) of the queries (fp16)
  __shared__ __align__(16) float sL[2][QTT];  // -lse * log2(e) of the tile's queries
  __shared__ __align__(16) float sDl[2][QTT];  // -D of the tile's queries
  // the task's raw k rows, for the dtheta terms of the epilogue (written and read by the same wave)
  __shared__ __align__(16) uint16_t sKraw[ROPE ? KTW * D : 8];
  __shared__ float sGmax[NW];
  extern __shared__ float2 sTab[];

  const int tid = threadIdx.x;
  Task T0;
  const int task = task_of_block(P, blockIdx.x);
  if (!decode_task(P, task, KTW, T0)) return;
  const TaskCtx X = make_ctx(P, T0, QTT);
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int M = P.M, n = X.n;
  const int TSTR = bwd_table_stride(M);  // cos/sin table row stride
  const float th_tab = ROPE ? theta[X.t.h * (D / 2) + (tid & 15)] : 0.f;  // the angle of this thread's table entries
  const int colstride = P.H * D, rowstride = P.Wg * colstride;
  // the largest output-gradient entry of the region: the query-tile kernel's entries of the
  // region's tiles (tasks task - qt .. task - qt + nqt - 1, which hold the same region and
  // head), reduced after the first barrier (see grad_scale_exp)
  float rmax = 0.f;
  for (int i = tid; i < X.t.nqt; i += NTHR) rmax = fmaxf(rmax, tmax[task - X.t.qt + i]);
  int gexp = 0;        // the region's gradient-scale exponent, set after the first barrier
  float gshift = 0.f;  // (float) gexp, added to the staged statistics

  // ---- this lane's keys: k (rotated, fp16) and v (bf16) as B operands; with a bias, the
  //      factor v_b as a k = 32 operand (rank 16: channels 0..15, zero-padded)
  u32x4 kraw[2], Vf[2], Vbf[2];
  int kpos_r[2], kpos_c[2];
  int64_t koffs[2];
  bool kvalid[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int ik = X.t.q0 + wave * 32 + 16 * a + c;  // the task's tile index counts keys here
    kvalid[a] = ik < n;
    int li = 0, lj = 0;
    if (kvalid[a]) split_idx(X, (uint32_t)ik, li, lj);
    kpos_r[a] = X.t.r0 + li;
    kpos_c[a] = X.t.c0 + lj;
    koffs[a] = X.img + X.regbase + li * rowstride + lj * colstride;
    if (kvalid[a]) {
      kraw[a] = *reinterpret_cast<const u32x4*>(k + koffs[a] + 8 * g);
      Vf[a] = *reinterpret_cast<const u32x4*>(v + koffs[a] + 8 * g);
    } else {
      kraw[a] = u32x4{0u, 0u, 0u, 0u};
      Vf[a] = u32x4{0u, 0u, 0u, 0u};
    }
    Vbf[a] = u32x4{0u, 0u, 0u, 0u};
    if (BIAS && kvalid[a] && (BR == 32 || g < 2)) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(
          bv + ((int64_t)X.t.h * M * M + kpos_r[a] * M + kpos_c[a]) * BR + 8 * g);
#pragma unroll
      for (int p = 0; p < 4; ++p) Vbf[a][p] = pack_f16(bf_lo(raw[p]), bf_hi(raw[p]));
    }
  }

  // ---- query tile loader: thread t owns chunk t % 4 of query t / 4 in q and dO (and, with a
  //      rank-32 bias, in the query's factor u); threads 0 .. QTT - 1 also stage query t's
  //      statistics; with rank 16, threads 0 .. 2 QTT - 1 the half t % 2 of the u of query t / 2
  const int lk = tid >> 2, lch = tid & 3;
  const int bk = BR == 32 ? lk : (tid % (2 * QTT)) >> 1, bch = BR == 32 ? lch : tid & 1;
  const bool bthread = BIAS && (BR == 32 || tid < 2 * QTT);
  Walker W, Ws, Wb;
  walker_init(W, X, lk, 8 * lch, rowstride, colstride);
  walker_init(Ws, X, tid < QTT ? tid : 0, 0, rowstride, colstride);
  walker_init(Wb, X, bk, 0, rowstride, colstride);
  // Every thread issues every load of the next tile, from an in-bounds address (threads past
  // the statistics or bias rows reload a valid row), and the arithmetic on the loaded values
  // waits until the tile is stored to LDS: with no branch around a load and no use right after
  // it, the loads of tile t + 1 stay in flight during the compute of tile t.
  u32x4 pq, po, pu = {0u, 0u, 0u, 0u};
  float pl = 0.f, pd = 0.f;
  bool psv = false;
  auto fetch = [&](int tile) {
    const bool valid = tile * QTT + lk < n;
    const int off = valid ? W.off : W.last;
    // rotated, scaled fp16 q and bf16 dO (times the gate) from the query-tile kernel
    pq = *reinterpret_cast<const u32x4*>(qt + X.img + off);
    po = *reinterpret_cast<const u32x4*>(dot + X.img + off);
    psv = tile * QTT + (tid < QTT ? tid : 0) < n;
    const int so = (psv ? Ws.off : Ws.last) / D;
    pl = lse[X.img / D + so];
    pd = delta[X.img / D + so];
    if (BIAS) {
      const int qn = (tile * QTT + bk < n) ? (X.t.r0 + Wb.ci) * M + (X.t.c0 + Wb.cj) : 0;
      pu = *reinterpret_cast<const u32x4*>(bu + ((int64_t)X.t.h * M * M + qn) * BR + 8 * bch);
    }
  };
  auto store = [&](int buf) {
    *reinterpret_cast<u32x4*>(&sQ[buf][lk * D + ((lch ^ kswz(lk)) * 8)]) = pq;
    *reinterpret_cast<u32x4*>(&sO[buf][lk * D + ((lch ^ vswz(lk)) * 8)]) = po;
    if (tid < QTT) {
      // a padded query gets the statistic +inf: its scores become -inf, so P = dS = 0
      sL[buf][tid] = psv ? gshift - pl * LOG2E : -INFINITY;  // P becomes 2^e P
      sDl[buf][tid] = -pd;
    }
    if (bthread) {
      u32x4 ur;
#pragma unroll
      for (int p = 0; p < 4; ++p) ur[p] = pack_f16(bf_lo(pu[p]) * LOG2E, bf_hi(pu[p]) * LOG2E);
      if (BR == 32)  // rows of 32 channels swizzled like Q
        *reinterpret_cast<u32x4*>(&sUb[buf][bk * 32 + 8 * (bch ^ kswz(bk))]) = ur;
      else
        *reinterpret_cast<u32x4*>(&sUb[buf][bk * 16 + 8 * (bch ^ bswz(bk))]) = ur;
    }
  };

  rmax = xmax32(xmax16(rmax));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o));
  if (lane == 0) sGmax[wave] = rmax;
  fetch(0);
  if (ROPE) build_rope_table<NTHR>(sTab, TSTR, th_tab, M, tid);
  __syncthreads();
  float gm = sGmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) gm = fmaxf(gm, sGmax[w]);
  gexp = grad_scale_exp(gm);  // one exponent for the region
  gshift = (float)gexp;
  u32x4 Kf[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (ROPE) *reinterpret_cast<u32x4*>(&sKraw[(wave * 32 + 16 * a + c) * D + 8 * g]) = kraw[a];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float x0 = bf_lo(kraw[a][p]), x1 = bf_hi(kraw[a][p]);
      if (ROPE) {
        const int j = 4 * g + p;
        const float2 t = sTab[j * TSTR + (j < D / 4 ? kpos_r[a] : kpos_c[a])];
        const float r0 = x0 * t.x - x1 * t.y, r1 = x0 * t.y + x1 * t.x;
        x0 = r0;
        x1 = r1;
      }
      Kf[a][p] = pack_f16(x0, x1);
    }
  }
  store(0);
  walker_advance(W, X);
  walker_advance(Ws, X);
  walker_advance(Wb, X);
  __syncthreads();

  const int krow = 8 * (c >> 2) + (c & 3);
  const int vrow = 8 * g + (c >> 2);
  const int vch = (c & 3) >> 1, vsub = 4 * (c & 1);
  f32x4 dV[2][2], dK[2][2];  // [dim / channel block][key block]
  f32x4 dVb[NBB][2];         // [bias channel block][key block]: channels 16 x + 4 g + e of key 16 a + c (times log2(e))
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int x = 0; x < NBB; ++x) dVb[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      dV[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
      dK[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const bool wave_live = X.t.q0 + wave * 32 < n;

  for (int tile = 0; tile < X.ntile; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < X.ntile;
    if (more) fetch(tile + 1);
    if (wave_live) {
      const int nst = min(QTT / 32, (n - tile * QTT + 31) / 32);
#pragma unroll
      for (int st = 0; st < QTT / 32; ++st) {
        if (st < nst) {
          const int qb = st * 32;
          u32x4 Qr[2], Or[2], OT[2], QTf[2], Ur[2], UT[NBB];
          f32x4 CL[2], CD[2];
          if (BIAS) {  // bias factor (u log2 e)^T: channel 16 x + c, queries qb + 8 g .. 8 g + 7
#pragma unroll
            for (int x = 0; x < NBB; ++x) {
              u32x2 h[2];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const int row = qb + vrow + 4 * hh;
                h[hh] = BR == 32 ? lds_read_tr16(&sUb[buf][row * 32 + (((2 * x + vch) ^ kswz(row)) * 8) + vsub])
                                 : lds_read_tr16(&sUb[buf][row * 16 + ((vch ^ bswz(row)) * 8) + vsub]);
              }
              UT[x] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
            }
          }
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int row = qb + krow + 4 * b;
            Qr[b] = *reinterpret_cast<const u32x4*>(&sQ[buf][row * D + ((g ^ kswz(row)) * 8)]);
            Or[b] = *reinterpret_cast<const u32x4*>(&sO[buf][row * D + ((g ^ vswz(row)) * 8)]);
            if (BR == 16) Ur[b] = *reinterpret_cast<const u32x4*>(&sUb[buf][row * 16 + 8 * ((g & 1) ^ bswz(row))]);
            if (BR == 32) Ur[b] = *reinterpret_cast<const u32x4*>(&sUb[buf][row * 32 + 8 * (g ^ kswz(row))]);
            // statistics of the accumulator rows of this lane: queries qb + 8 g + 4 b + e
            CL[b] = *reinterpret_cast<const f32x4*>(&sL[buf][qb + 8 * g + 4 * b]);
            CD[b] = *reinterpret_cast<const f32x4*>(&sDl[buf][qb + 8 * g + 4 * b]);
          }
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            u32x2 h[2], hq[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int row = qb + vrow + 4 * hh;
              h[hh] = lds_read_tr16(&sO[buf][row * D + (((2 * x + vch) ^ vswz(row)) * 8) + vsub]);
              hq[hh] = lds_read_tr16(&sQ[buf][row * D + (((2 * x + vch) ^ kswz(row)) * 8) + vsub]);
            }
            OT[x] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
            QTf[x] = u32x4{hq[0][0], hq[0][1], hq[1][0], hq[1][1]};
          }
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            f32x4 S[2], G[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              // rows: queries, column: key 16 a + c (bias channels first, as in the forward pass)
              S[b] = BIAS ? mfma16_f16(Ur[b], Vbf[a], CL[b]) : CL[b];
              S[b] = mfma16_f16(Qr[b], Kf[a], S[b]);
              G[b] = mfma16_bf16(Or[b], Vf[a], CD[b]);  // dP - D
            }
            uint32_t Pb[4], dS16[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int b = t >> 1, e0 = 2 * (t & 1);
              const float p0 = __builtin_amdgcn_exp2f(S[b][e0]), p1 = __builtin_amdgcn_exp2f(S[b][e0 + 1]);
              Pb[t] = pack_bf16(p0, p1);
              dS16[t] = pack_f16(p0 * G[b][e0], p1 * G[b][e0 + 1]);
            }
            const u32x4 Pa = {Pb[0], Pb[1], Pb[2], Pb[3]}, dSa = {dS16[0], dS16[1], dS16[2], dS16[3]};
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              dV[x][a] = mfma16_bf16(OT[x], Pa, dV[x][a]);
              dK[x][a] = mfma16_f16(QTf[x], dSa, dK[x][a]);
            }
#pragma unroll
            for (int x = 0; x < NBB; ++x)
              if (BIAS) dVb[x][a] = mfma16_f16(UT[x], dSa, dVb[x][a]);
          }
        }
      }
    }
    if (more) {
      store(buf ^ 1);
      walker_advance(W, X);
      walker_advance(Ws, X);
      walker_advance(Wb, X);
    }
    __syncthreads();
  }

  // ---- the gradient of the bias factor v_b (shared by every window and image: added into its
  //      window position with atomics; the u tile carried log2(e)), all products unscaled by 2^-e
  const float gunscale = __builtin_ldexpf(1.0f, -gexp), gunscale_ln2 = gunscale * LN2;
  if (BIAS) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (!kvalid[a]) continue;
      float* dst = dbv + ((int64_t)X.t.h * M * M + kpos_r[a] * M + kpos_c[a]) * BR + 4 * g;
#pragma unroll
      for (int x = 0; x < NBB; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(dst + 16 * x + e, dVb[x][a][e] * gunscale_ln2);
    }
  }

  // ---- epilogue: dv, dk = R^T (dS^T Q~) ln 2, and the k part of dtheta (the raw k channels
  //      of the dtheta sums from LDS, where the prologue left them)
  u32x2 kr2[2][2] = {};
  if (ROPE) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        kr2[a][x] = *reinterpret_cast<const u32x2*>(&sKraw[(wave * 32 + 16 * a + c) * D + 16 * x + 4 * g]);
  }
  float dth[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // [channel block][pair]: this lane's angle-gradient terms
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (!kvalid[a]) continue;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      *reinterpret_cast<float4*>(dv + koffs[a] + 16 * x + 4 * g) =
          make_float4(dV[x][a][0] * gunscale, dV[x][a][1] * gunscale, dV[x][a][2] * gunscale,
                      dV[x][a][3] * gunscale);
      float r4[4];
      const int pos = x == 0 ? kpos_r[a] : kpos_c[a];
      finish_grad4<ROPE>(dK[x][a], gunscale_ln2, 8 * x + 2 * g, pos, sTab, TSTR, kr2[a][x], dth[x], r4);
      *reinterpret_cast<float4*>(dk + koffs[a] + 16 * x + 4 * g) = make_float4(r4[0], r4[1], r4[2], r4[3]);
    }
  }
  if (ROPE) dtheta_flush<NW>(dth, dth_part, X.t.h, P.H, tid);
}

// ---- Kernel C: the whole backward pass of one wrap region of at most 64 tokens (window side
//      M <= 8) and one head, in a workgroup of two waves.  The region's K, V, Q~ and dO~ sit
//      in LDS at once.  Phase A does the query-tile kernel's work for the region's queries
//      (wave w: queries 32 w .. 32 w + 31) against every key and leaves P and dS of each pair
//      in LDS, [query][key]; phase B does the key-tile kernel's products (wave w: keys
//      32 w .. 32 w + 31) with P and dS read back transposed.  The scores, dP and the
//      exponentials are computed once per pair, nothing is staged in memory, and every sum
//      (dq over the region's keys; dk, dv over its queries) is complete inside the workgroup.
//      The gradient scale: per query row for dq and dU, as in kernel A; one per region (the
//      workgroup's largest output-gradient entry) for the P and dS that phase B consumes.
constexpr int SMALL_REGION = 64;  // tokens of a region the fused kernel holds (every region at M <= 8)
// 16-byte chunk swizzle of the [query][key] P and dS tiles (rows of 64 entries, 8 chunks)
__device__ __forceinline__ int pswz(int row) { return row & 7; }

// Two waves per SIMD: its 34-42 KB of LDS allow four workgroups per CU.
template <bool ROPE, bool OUTF32, int BR, bool GATE>
__global__ __launch_bounds__(128, 2) void wattn_bwd_small_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ out, const void* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dth_part,
    const float* __restrict__ theta, const uint16_t* __restrict__ bu, const uint16_t* __restrict__ bv,
    float* __restrict__ dbu, float* __restrict__ dbv, const uint16_t* __restrict__ gz, float* __restrict__ dz,
    const WattnPlan P) {
  constexpr int NW = 2, NTHR = 64 * NW, NR = SMALL_REGION;
  constexpr bool BIAS = BR > 0;
  constexpr int NBB = BR == 32 ? 2 : 1;  // 16-channel blocks of the bias gradient
  static_assert(BR == 0 || BR == 16 || BR == 32, "bias rank 0, 16 or 32");
  static_assert(NR == 32 * NW, "one query and one key block of 32 per wave");
  __shared__ __align__(16) uint16_t sK[NR * D];   // rotated k, fp16
  __shared__ __align__(16) uint16_t sV[NR * D];   // v, bf16
  __shared__ __align__(16) uint16_t sQ[NR * D];   // rotated q times log2(e) / sqrt(d), fp16
  __shared__ __align__(16) uint16_t sO[NR * D];   // dO (times the gate), bf16
  __shared__ __align__(16) uint16_t sP[NR * NR];  // 2^e P, bf16, [query][key]
  __shared__ __align__(16) uint16_t sS[NR * NR];  // 2^e dS, fp16, [query][key]
  __shared__ __align__(16) uint16_t sKb[BIAS ? NR * BR : 8];  // bias factor v of the keys (fp16)
  __shared__ __align__(16) uint16_t sUb[BIAS ? NR * BR : 8];  // u log2(e) of the queries (fp16)
  __shared__ float sGmax[NW];
  extern __shared__ float2 sTab[];

  const int tid = threadIdx.x;
  Task T0;
  if (!decode_task(P, task_of_block(P, blockIdx.x), NR, T0)) return;
  const TaskCtx X = make_ctx(P, T0, NR);
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int M = P.M, n = X.n;  // n <= NR
  const int TSTR = bwd_table_stride(M);  // cos/sin table row stride
  const float th_tab = ROPE ? theta[X.t.h * (D / 2) + (tid & 15)] : 0.f;  // the angle of this thread's table entries
  const int colstride = P.H * D, rowstride = P.Wg * colstride;
  float dth[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // this lane's angle-gradient terms, both phases

  // ---- this lane's queries 32 wave + 16 a + c, channels 8 g .. 8 g + 7 (as in kernel A); all
  //      loads first, from valid addresses
  u32x4 qraw[2], dOf[2], Qb[2];
  f32x4 CnL[2], CnD[2];
  int qpos_r[2], qpos_c[2];
  int64_t qoff[2];
  bool qvalid[2];
  float go[2][8], o[2][8], lraw[2];
  u32x4 zraw[2], braw[2];
  // raw q and k channels 16 cb + 4 g .. + 3 of the lane's rows, for the dtheta terms of the two
  // epilogues (the wave's keys are its queries' tokens); loaded with the rest, kept in registers
  u32x2 qr2[2][2] = {}, kr2[2][2] = {};
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int iq = wave * 32 + 16 * a + c;
    qvalid[a] = iq < n;
    int li = 0, lj = 0;
    if (qvalid[a]) split_idx(X, (uint32_t)iq, li, lj);
    qpos_r[a] = X.t.r0 + li;
    qpos_c[a] = X.t.c0 + lj;
    qoff[a] = X.img + X.regbase + li * rowstride + lj * colstride;
    qraw[a] = *reinterpret_cast<const u32x4*>(q + qoff[a] + 8 * g);
    load8<OUTF32>(dout, qoff[a] + 8 * g, go[a]);
    load8<OUTF32>(out, qoff[a] + 8 * g, o[a]);
    lraw[a] = lse[qoff[a] / D];
    if (GATE) zraw[a] = *reinterpret_cast<const u32x4*>(gz + qoff[a] + 8 * g);
    if (BIAS)
      braw[a] = *reinterpret_cast<const u32x4*>(
          bu + ((int64_t)X.t.h * M * M + qpos_r[a] * M + qpos_c[a]) * BR + 8 * (BR == 32 ? g : (g & 1)));
    if (ROPE) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        qr2[a][cb] = *reinterpret_cast<const u32x2*>(q + qoff[a] + 16 * cb + 4 * g);
        kr2[a][cb] = *reinterpret_cast<const u32x2*>(k + qoff[a] + 16 * cb + 4 * g);
      }
    }
  }
  // ---- the region's keys: thread t stages chunk t % 4 of keys t / 4 and t / 4 + 32 (keys past
  //      the region end repeat its last key: finite data whose scores are masked), and the same
  //      quarter of their bias-factor rows
  const int lk = tid >> 2, lch = tid & 3;
  u32x4 pk[2], pv[2], pb[2];
  int lpos[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int key = lk + 32 * j;
    int li, lj;
    split_idx(X, (uint32_t)min(key, n - 1), li, lj);
    const uint32_t off = (uint32_t)(X.regbase + li * rowstride + lj * colstride + 8 * lch) * 2u;
    pk[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(k + X.img) + off);
    pv[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(v + X.img) + off);
    lpos[j] = (lch < 2) ? (X.t.r0 + li) : (X.t.c0 + lj);
    pb[j] = u32x4{0u, 0u, 0u, 0u};
    if (BIAS) {
      const uint16_t* src = bv + ((int64_t)X.t.h * M * M + (X.t.r0 + li) * M + (X.t.c0 + lj)) * BR + (BR / 4) * lch;
      if (BR == 16) {
        const u32x2 h = *reinterpret_cast<const u32x2*>(src);
        pb[j] = u32x4{h[0], h[1], 0u, 0u};
      } else {
        pb[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  }

  // ---- per query row: D, the gate, the row's scale exponent, the operands
  int gexp[2];
  float wgmax = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float Dp = 0.f, L2 = 0.f;
    if (qvalid[a]) {
      L2 = lraw[a] * LOG2E;
      if (GATE) {  // as in kernel A: dO becomes dout * sigmoid(z), dz = dout * out * (1 - sigmoid(z))
#pragma unroll
        for (int e = 0; e < 8; ++e) Dp += go[a][e] * o[a][e];
        float gzv[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float s0 = sigmoidf_fast(bf_lo(zraw[a][p])), s1 = sigmoidf_fast(bf_hi(zraw[a][p]));
          gzv[2 * p] = go[a][2 * p] * o[a][2 * p] * (1.0f - s0);
          gzv[2 * p + 1] = go[a][2 * p + 1] * o[a][2 * p + 1] * (1.0f - s1);
          go[a][2 * p] *= s0;
          go[a][2 * p + 1] *= s1;
        }
        float* dst = dz + qoff[a] + 8 * g;
        *reinterpret_cast<float4*>(dst) = make_float4(gzv[0], gzv[1], gzv[2], gzv[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(gzv[4], gzv[5], gzv[6], gzv[7]);
      }
    } else {
      qraw[a] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) go[a][e] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) dOf[a][p] = pack_bf16(go[a][2 * p], go[a][2 * p + 1]);
    if (!GATE && qvalid[a]) {  // D from the bf16 dO that dP uses (as in kernel A)
#pragma unroll
      for (int p = 0; p < 4; ++p) Dp += bf_lo(dOf[a][p]) * o[a][2 * p] + bf_hi(dOf[a][p]) * o[a][2 * p + 1];
    }
    const float Dn = xsum32(xsum16(Dp));
    float gm = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) gm = fmaxf(gm, fabsf(go[a][e]));
    gm = xmax32(xmax16(gm));
    wgmax = fmaxf(wgmax, gm);
    gexp[a] = grad_scale_exp(gm);
    // a padded query gets -inf: its P and dS are exactly 0, in LDS too
    const float cl = qvalid[a] ? (float)gexp[a] - L2 : -INFINITY;
    Qb[a] = u32x4{0u, 0u, 0u, 0u};
    if (BIAS && qvalid[a] && (BR == 32 || g < 2)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) Qb[a][p] = pack_f16(bf_lo(braw[a][p]) * LOG2E, bf_hi(braw[a][p]) * LOG2E);
    }
    CnL[a] = f32x4{cl, cl, cl, cl};
    CnD[a] = f32x4{-Dn, -Dn, -Dn, -Dn};
  }
  {
    float wm = wgmax;
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) wm = fmaxf(wm, __shfl_xor(wm, s));
    if (lane == 0) sGmax[wave] = wm;
  }
  if (ROPE) build_rope_table<NTHR>(sTab, TSTR, th_tab, M, tid);
  __syncthreads();
  const int ereg = grad_scale_exp(fmaxf(sGmax[0], sGmax[1]));  // the region's exponent

  // ---- LDS: rotated keys (fp16), values, bias factors of the keys; the lane's rotated, scaled
  //      queries (fp16), dO~ (bf16) and u log2(e) (fp16) for phase B
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int key = lk + 32 * j;
    u32x4 kr;
    const int lp = min(lpos[j], M - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = bf_lo(pk[j][p]), x1 = bf_hi(pk[j][p]);
      if (ROPE) {
        const float2 t = sTab[(4 * lch + p) * TSTR + lp];
        kr[p] = pack_f16(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
      } else {
        kr[p] = pack_f16(x0, x1);
      }
    }
    *reinterpret_cast<u32x4*>(&sK[key * D + ((lch ^ kswz(key)) * 8)]) = kr;
    *reinterpret_cast<u32x4*>(&sV[key * D + ((lch ^ vswz(key)) * 8)]) = pv[j];
    if (BR == 16) {
      const u32x2 br = {pack_f16(bf_lo(pb[j][0]), bf_hi(pb[j][0])), pack_f16(bf_lo(pb[j][1]), bf_hi(pb[j][1]))};
      *reinterpret_cast<u32x2*>(&sKb[key * 16 + 8 * ((lch >> 1) ^ bswz(key)) + 4 * (lch & 1)]) = br;
    }
    if (BR == 32) {
      u32x4 br;
#pragma unroll
      for (int p = 0; p < 4; ++p) br[p] = pack_f16(bf_lo(pb[j][p]), bf_hi(pb[j][p]));
      *reinterpret_cast<u32x4*>(&sKb[key * 32 + 8 * (lch ^ kswz(key))]) = br;
    }
  }
  u32x4 Qf[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const float qscale = LOG2E * 0.17677669529663687f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float x0 = bf_lo(qraw[a][p]), x1 = bf_hi(qraw[a][p]);
      if (ROPE) {
        const int j = 4 * g + p;
        const float2 t = sTab[j * TSTR + (j < D / 4 ? qpos_r[a] : qpos_c[a])];
        const float r0 = x0 * t.x - x1 * t.y, r1 = x0 * t.y + x1 * t.x;
        x0 = r0;
        x1 = r1;
      }
      Qf[a][p] = pack_f16(x0 * qscale, x1 * qscale);
    }
    const int qi = wave * 32 + 16 * a + c;  // padded queries store zeros
    *reinterpret_cast<u32x4*>(&sQ[qi * D + ((g ^ kswz(qi)) * 8)]) = Qf[a];
    *reinterpret_cast<u32x4*>(&sO[qi * D + ((g ^ vswz(qi)) * 8)]) = dOf[a];
    if (BR == 16 && g < 2) *reinterpret_cast<u32x4*>(&sUb[qi * 16 + 8 * (g ^ bswz(qi))]) = Qb[a];
    if (BR == 32) *reinterpret_cast<u32x4*>(&sUb[qi * 32 + 8 * (g ^ kswz(qi))]) = Qb[a];
  }
  __syncthreads();

  const int krow = 8 * (c >> 2) + (c & 3);
  const int vrow = 8 * g + (c >> 2);
  const int vch = (c & 3) >> 1, vsub = 4 * (c & 1);
  const bool wave_live = wave * 32 < n;

  // ---- phase A: dq (and dU) of the wave's queries over all keys; P and dS to LDS
  if (wave_live) {
    f32x4 dQ[2][2], dU[NBB][2];
    float fscale[2];  // 2^(ereg - gexp): from the row's scale to the region's
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      dQ[0][a] = f32x4{0.f, 0.f, 0.f, 0.f};
      dQ[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < NBB; ++cb) dU[cb][a] = f32x4{0.f, 0.f, 0.f, 0.f};
      fscale[a] = __builtin_ldexpf(1.0f, ereg - gexp[a]);
    }
    auto kblock = [&](int kb, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      u32x4 Kf[2], Vr[2], KTf[2], Kb[2], VbT[NBB];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int key = kb + krow + 4 * b;
        Kf[b] = *reinterpret_cast<const u32x4*>(&sK[key * D + ((g ^ kswz(key)) * 8)]);
        Vr[b] = *reinterpret_cast<const u32x4*>(&sV[key * D + ((g ^ vswz(key)) * 8)]);
        if (BR == 16) Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[key * 16 + 8 * ((g & 1) ^ bswz(key))]);
        if (BR == 32) Kb[b] = *reinterpret_cast<const u32x4*>(&sKb[key * 32 + 8 * (g ^ kswz(key))]);
      }
      if (BIAS) {
#pragma unroll
        for (int cb = 0; cb < NBB; ++cb) {
          u32x2 h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = kb + vrow + 4 * hh;
            h[hh] = BR == 32 ? lds_read_tr16(&sKb[row * 32 + (((2 * cb + vch) ^ kswz(row)) * 8) + vsub])
                             : lds_read_tr16(&sKb[row * 16 + ((vch ^ bswz(row)) * 8) + vsub]);
          }
          VbT[cb] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
        }
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        u32x2 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = kb + vrow + 4 * hh;
          h[hh] = lds_read_tr16(&sK[row * D + (((2 * cb + vch) ^ kswz(row)) * 8) + vsub]);
        }
        KTf[cb] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        f32x4 S[2], G[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          S[b] = BIAS ? mfma16_f16(Kb[b], Qb[a], CnL[a]) : CnL[a];
          S[b] = mfma16_f16(Kf[b], Qf[a], S[b]);
          G[b] = mfma16_bf16(Vr[b], dOf[a], CnD[a]);  // dP - D
        }
        uint32_t dS16[4], Pr[4], Sr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int b = t >> 1, e0 = 2 * (t & 1);
          float s0 = S[b][e0], s1 = S[b][e0 + 1];
          if (MASK) {
            if (kb + 8 * g + 4 * b + e0 >= n) s0 = -INFINITY;
            if (kb + 8 * g + 4 * b + e0 + 1 >= n) s1 = -INFINITY;
          }
          const float p0 = __builtin_amdgcn_exp2f(s0), p1 = __builtin_amdgcn_exp2f(s1);
          const float d0 = p0 * G[b][e0], d1 = p1 * G[b][e0 + 1];
          dS16[t] = pack_f16(d0, d1);
          Pr[t] = pack_bf16(p0 * fscale[a], p1 * fscale[a]);
          Sr[t] = pack_f16(d0 * fscale[a], d1 * fscale[a]);
        }
        const u32x4 dSa = {dS16[0], dS16[1], dS16[2], dS16[3]};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) dQ[cb][a] = mfma16_f16(KTf[cb], dSa, dQ[cb][a]);
#pragma unroll
        for (int cb = 0; cb < NBB; ++cb)
          if (BIAS) dU[cb][a] = mfma16_f16(VbT[cb], dSa, dU[cb][a]);
        // keys kb + 8 g .. kb + 8 g + 7 of query qi: one 16-byte chunk of its P and dS rows
        const int qi = wave * 32 + 16 * a + c;
        const int ch = ((kb >> 3) + g) ^ pswz(qi);
        *reinterpret_cast<u32x4*>(&sP[qi * NR + 8 * ch]) = u32x4{Pr[0], Pr[1], Pr[2], Pr[3]};
        *reinterpret_cast<u32x4*>(&sS[qi * NR + 8 * ch]) = u32x4{Sr[0], Sr[1], Sr[2], Sr[3]};
      }
    };
#pragma unroll
    for (int st = 0; st < NR / 32; ++st) {
      const int kb = st * 32;
      if (kb + 32 <= n)
        kblock(kb, std::false_type{});
      else if (kb < n)
        kblock(kb, std::true_type{});
    }
    // epilogue of phase A: dU, dq and the q part of dtheta (as in kernel A)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (!qvalid[a]) continue;
      if (BIAS) {
        float* dst = dbu + ((int64_t)X.t.h * M * M + qpos_r[a] * M + qpos_c[a]) * BR + 4 * g;
        const float us = __builtin_ldexpf(1.0f, -gexp[a]);
#pragma unroll
        for (int cb = 0; cb < NBB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(dst + 16 * cb + e, dU[cb][a][e] * us);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float r4[4];
        const int pos = cb == 0 ? qpos_r[a] : qpos_c[a];
        finish_grad4<ROPE>(dQ[cb][a], __builtin_ldexpf(0.17677669529663687f, -gexp[a]), 8 * cb + 2 * g, pos, sTab,
                           TSTR, qr2[a][cb], dth[cb], r4);
        *reinterpret_cast<float4*>(dq + qoff[a] + 16 * cb + 4 * g) = make_float4(r4[0], r4[1], r4[2], r4[3]);
      }
    }
  }
  __syncthreads();

  // ---- phase B: dv, dk (and dV_b) of the wave's keys 32 wave + 16 a + c over all queries
  if (wave_live) {
    f32x4 dV[2][2], dK[2][2], dVb[NBB][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        dV[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
        dK[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int x = 0; x < NBB; ++x) dVb[x][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int st = 0; st < NR / 32; ++st) {
      const int qb = st * 32;
      if (qb < n) {
        u32x4 OT[2], QTf[2], UT[NBB];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          u32x2 h[2], hq[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = qb + vrow + 4 * hh;
            h[hh] = lds_read_tr16(&sO[row * D + (((2 * x + vch) ^ vswz(row)) * 8) + vsub]);
            hq[hh] = lds_read_tr16(&sQ[row * D + (((2 * x + vch) ^ kswz(row)) * 8) + vsub]);
          }
          OT[x] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
          QTf[x] = u32x4{hq[0][0], hq[0][1], hq[1][0], hq[1][1]};
        }
        if (BIAS) {
#pragma unroll
          for (int x = 0; x < NBB; ++x) {
            u32x2 h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int row = qb + vrow + 4 * hh;
              h[hh] = BR == 32 ? lds_read_tr16(&sUb[row * 32 + (((2 * x + vch) ^ kswz(row)) * 8) + vsub])
                               : lds_read_tr16(&sUb[row * 16 + ((vch ^ bswz(row)) * 8) + vsub]);
            }
            UT[x] = u32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
          }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          // B operands: key column 32 wave + 16 a + c, queries qb + 8 g .. qb + 8 g + 7
          const int kch = 2 * (2 * wave + a) + vch;  // 8-key chunk of the column
          u32x2 hp[2], hs[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = qb + vrow + 4 * hh;
            hp[hh] = lds_read_tr16(&sP[row * NR + ((kch ^ pswz(row)) * 8) + vsub]);
            hs[hh] = lds_read_tr16(&sS[row * NR + ((kch ^ pswz(row)) * 8) + vsub]);
          }
          const u32x4 Pa = {hp[0][0], hp[0][1], hp[1][0], hp[1][1]};
          const u32x4 dSa = {hs[0][0], hs[0][1], hs[1][0], hs[1][1]};
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            dV[x][a] = mfma16_bf16(OT[x], Pa, dV[x][a]);
            dK[x][a] = mfma16_f16(QTf[x], dSa, dK[x][a]);
          }
#pragma unroll
          for (int x = 0; x < NBB; ++x)
            if (BIAS) dVb[x][a] = mfma16_f16(UT[x], dSa, dVb[x][a]);
        }
      }
    }
    // epilogue of phase B: dV_b, dv, dk and the k part of dtheta (as in kernel B)
    const float gunscale = __builtin_ldexpf(1.0f, -ereg), gunscale_ln2 = gunscale * LN2;
    // the wave's keys are the tokens of its queries: the same offsets, positions and validity
    const int64_t* koffs = qoff;
    const int* kpos_r = qpos_r;
    const int* kpos_c = qpos_c;
    const bool* kvalid = qvalid;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (!kvalid[a]) continue;
      if (BIAS) {
        float* dst = dbv + ((int64_t)X.t.h * M * M + kpos_r[a] * M + kpos_c[a]) * BR + 4 * g;
#pragma unroll
        for (int x = 0; x < NBB; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(dst + 16 * x + e, dVb[x][a][e] * gunscale_ln2);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        *reinterpret_cast<float4*>(dv + koffs[a] + 16 * x + 4 * g) =
            make_float4(dV[x][a][0] * gunscale, dV[x][a][1] * gunscale, dV[x][a][2] * gunscale,
                        dV[x][a][3] * gunscale);
        float r4[4];
        const int pos = x == 0 ? kpos_r[a] : kpos_c[a];
        finish_grad4<ROPE>(dK[x][a], gunscale_ln2, 8 * x + 2 * g, pos, sTab, TSTR, kr2[a][x], dth[x], r4);
        *reinterpret_cast<float4*>(dk + koffs[a] + 16 * x + 4 * g) = make_float4(r4[0], r4[1], r4[2], r4[3]);
      }
    }
  }
  if (ROPE) dtheta_flush<NW>(dth, dth_part, X.t.h, P.H, tid);
}

// zeroes up to three float arrays in one launch (the backward pass's atomic targets), so that
// the clearing costs one dispatch however many of them a call has
struct ZeroList {
  float* p[3];
  int n[3];
};
__global__ void wattn_fill_zero_kernel(const ZeroList z) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (i < z.n[j]) z.p[j][i] = 0.f;
}

// dtheta[i] = the sum of the WATTN_DTHETA_COPIES partial sums of entry i (n = H * d / 2 entries):
// one workgroup of WATTN_DTHETA_COPIES threads per entry, thread c loads copy c, a fixed-order
// tree sum (shuffles within the waves, then over the waves)
static_assert(WATTN_DTHETA_COPIES == 256, "one 256-thread workgroup per dtheta entry");
__global__ __launch_bounds__(WATTN_DTHETA_COPIES) void wattn_dtheta_reduce_kernel(const float* __restrict__ part,
                                                                                float* __restrict__ dtheta, int n) {
  __shared__ float sw[WATTN_DTHETA_COPIES / 64];
  const int i = blockIdx.x, t = threadIdx.x;
  float v = part[(int64_t)t * n + i];
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) v += __shfl_xor(v, s);
  if ((t & 63) == 0) sw[t >> 6] = v;
  __syncthreads();
  if (t == 0) dtheta[i] = (sw[0] + sw[1]) + (sw[2] + sw[3]);
}

}  // namespace

// ------------------------------------------------------------------------------------
// Launchers (C++ linkage, internal to the library)
// ------------------------------------------------------------------------------------

template <int NW, int NKS, bool ROPE, bool OUTF32, bool GATE>
static hipError_t launch_bf16_inst(const WattnPlan& plan, const void* q, const void* k, const void* v, void* out,
                                   const float* theta, const void* bu, const void* bv, float* lse, const void* gz,
                                   hipStream_t stream) {
  if (ROPE && plan.M > table_stride(NW)) return hipErrorInvalidValue;
  const size_t table_bytes = ROPE ? (size_t)table_stride(NW) * (D / 2) * sizeof(float2) : 0;
  hipLaunchKernelGGL((wattn_fwd_bf16_kernel<NW, NKS, ROPE, OUTF32, GATE>), dim3(plan.grid), dim3(64 * NW),
                     table_bytes, stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), out, theta, static_cast<const uint16_t*>(bu),
                     static_cast<const uint16_t*>(bv), lse, static_cast<const uint16_t*>(gz), plan);
  return hipGetLastError();
}

template <int NW, bool GATE>
static hipError_t launch_bf16_nw(const WattnPlan& plan, int nks, bool rope, bool out_f32, const void* q,
                                 const void* k, const void* v, void* out, const float* theta, const void* bu,
                                 const void* bv, float* lse, const void* gz, hipStream_t stream) {
#define WATTN_FWD_ARGS plan, q, k, v, out, theta, bu, bv, lse, gz, stream
  const int sel = (nks - 2) * 4 + (rope ? 2 : 0) + (out_f32 ? 1 : 0);
  switch (sel) {
    case 0: return launch_bf16_inst<NW, 2, false, false, GATE>(WATTN_FWD_ARGS);
    case 1: return launch_bf16_inst<NW, 2, false, true, GATE>(WATTN_FWD_ARGS);
    case 2: return launch_bf16_inst<NW, 2, true, false, GATE>(WATTN_FWD_ARGS);
    case 3: return launch_bf16_inst<NW, 2, true, true, GATE>(WATTN_FWD_ARGS);
    case 4: return launch_bf16_inst<NW, 3, false, false, GATE>(WATTN_FWD_ARGS);
    case 5: return launch_bf16_inst<NW, 3, false, true, GATE>(WATTN_FWD_ARGS);
    case 6: return launch_bf16_inst<NW, 3, true, false, GATE>(WATTN_FWD_ARGS);
    case 7: return launch_bf16_inst<NW, 3, true, true, GATE>(WATTN_FWD_ARGS);
    case 8: return launch_bf16_inst<NW, 4, false, false, GATE>(WATTN_FWD_ARGS);
    case 9: return launch_bf16_inst<NW, 4, false, true, GATE>(WATTN_FWD_ARGS);
    case 10: return launch_bf16_inst<NW, 4, true, false, GATE>(WATTN_FWD_ARGS);
    case 11: return launch_bf16_inst<NW, 4, true, true, GATE>(WATTN_FWD_ARGS);
    default: return hipErrorInvalidValue;
  }
#undef WATTN_FWD_ARGS
}

template <bool GATE>
static hipError_t launch_bf16_gate(const WattnPlan& plan, int nks, bool rope, bool out_f32, const void* q,
                                   const void* k, const void* v, void* out, const float* theta, const void* bu,
                                   const void* bv, float* lse, const void* gz, hipStream_t stream) {
  switch (plan.nw) {
    case 2: return launch_bf16_nw<2, GATE>(plan, nks, rope, out_f32, q, k, v, out, theta, bu, bv, lse, gz, stream);
    case 4: return launch_bf16_nw<4, GATE>(plan, nks, rope, out_f32, q, k, v, out, theta, bu, bv, lse, gz, stream);
    case 8: return launch_bf16_nw<8, GATE>(plan, nks, rope, out_f32, q, k, v, out, theta, bu, bv, lse, gz, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t wattn_launch_bf16(const WattnPlan& plan, int nks, bool rope, bool out_f32, const void* q,
                             const void* k, const void* v, void* out, const float* theta, const void* bu,
                             const void* bv, float* lse, const void* gz, hipStream_t stream) {
  return gz != nullptr ? launch_bf16_gate<true>(plan, nks, rope, out_f32, q, k, v, out, theta, bu, bv, lse, gz, stream)
                       : launch_bf16_gate<false>(plan, nks, rope, out_f32, q, k, v, out, theta, bu, bv, lse, gz, stream);
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
  else if (r == 32)
    hipLaunchKernelGGL((wattn_fwd_f32_kernel<32>), grid, block, 0, stream, Q, K, V, O, theta, U, W, plan);
  else
    hipLaunchKernelGGL((wattn_fwd_f32_kernel<0>), grid, block, 0, stream, Q, K, V, O, theta, U, W, plan);
  return hipGetLastError();
}

// ---- backward launchers
template <int NW, bool ROPE, bool OUTF32, int BR, bool GATE>
static hipError_t launch_bwd_inst(const WattnPlan& plan, const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, float* delta, float* dq, float* dk, float* dv,
                                  float* dtheta, const float* theta, const void* bu, const void* bv, float* dbu,
                                  float* dbv, const void* gz, float* dz, uint16_t* qt, uint16_t* dot,
                                  float* tmax, hipStream_t stream) {
  const size_t table_bytes = ROPE ? (size_t)bwd_table_stride(plan.M) * (D / 2) * sizeof(float2) : 0;
  auto Q = static_cast<const uint16_t*>(q);
  auto K = static_cast<const uint16_t*>(k);
  auto V = static_cast<const uint16_t*>(v);
  auto BU = static_cast<const uint16_t*>(bu);
  auto BV = static_cast<const uint16_t*>(bv);
  auto GZ = static_cast<const uint16_t*>(gz);
  hipLaunchKernelGGL((wattn_bwd_dq_kernel<NW, ROPE, OUTF32, BR, GATE>), dim3(plan.grid), dim3(64 * NW),
                     table_bytes, stream, Q, K, V, out, dout, lse, delta, dq, dtheta, theta, BU, BV, dbu, GZ, dz, qt,
                     dot, tmax, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((wattn_bwd_dkdv_kernel<NW, ROPE, BR>), dim3(plan.grid), dim3(64 * NW), table_bytes, stream,
                     static_cast<const uint16_t*>(qt), K, V, static_cast<const uint16_t*>(dot), lse,
                     static_cast<const float*>(delta), dk, dv, dtheta, theta, BU, BV, dbv,
                     static_cast<const float*>(tmax), plan);
  return hipGetLastError();
}

// the fused kernel of regions of at most 64 tokens (window side M <= 8)
template <bool ROPE, bool OUTF32, int BR, bool GATE>
static hipError_t launch_small_inst(const WattnPlan& plan, const void* q, const void* k, const void* v,
                                    const void* out, const void* dout, const float* lse, float* dq, float* dk,
                                    float* dv, float* dtheta, const float* theta, const void* bu, const void* bv,
                                    float* dbu, float* dbv, const void* gz, float* dz, hipStream_t stream) {
  if (plan.nw != 2 || plan.M * plan.M > SMALL_REGION) return hipErrorInvalidValue;
  const size_t table_bytes = ROPE ? (size_t)bwd_table_stride(plan.M) * (D / 2) * sizeof(float2) : 0;
  hipLaunchKernelGGL((wattn_bwd_small_kernel<ROPE, OUTF32, BR, GATE>), dim3(plan.grid), dim3(128), table_bytes,
                     stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), out, dout, lse, dq, dk, dv, dtheta, theta,
                     static_cast<const uint16_t*>(bu), static_cast<const uint16_t*>(bv), dbu, dbv,
                     static_cast<const uint16_t*>(gz), dz, plan);
  return hipGetLastError();
}

template <bool GATE>
static hipError_t launch_small(const WattnPlan& plan, bool rope, bool out_f32, int br, const void* q, const void* k,
                               const void* v, const void* out, const void* dout, const float* lse, float* dq,
                               float* dk, float* dv, float* dtheta, const float* theta, const void* bu,
                               const void* bv, float* dbu, float* dbv, const void* gz, float* dz,
                               hipStream_t stream) {
#define WATTN_SMALL_ARGS plan, q, k, v, out, dout, lse, dq, dk, dv, dtheta, theta, bu, bv, dbu, dbv, gz, dz, stream
  const int sel = (br / 16) * 4 + (rope ? 2 : 0) + (out_f32 ? 1 : 0);
  switch (sel) {
    case 0: return launch_small_inst<false, false, 0, GATE>(WATTN_SMALL_ARGS);
    case 1: return launch_small_inst<false, true, 0, GATE>(WATTN_SMALL_ARGS);
    case 2: return launch_small_inst<true, false, 0, GATE>(WATTN_SMALL_ARGS);
    case 3: return launch_small_inst<true, true, 0, GATE>(WATTN_SMALL_ARGS);
    case 4: return launch_small_inst<false, false, 16, GATE>(WATTN_SMALL_ARGS);
    case 5: return launch_small_inst<false, true, 16, GATE>(WATTN_SMALL_ARGS);
    case 6: return launch_small_inst<true, false, 16, GATE>(WATTN_SMALL_ARGS);
    case 7: return launch_small_inst<true, true, 16, GATE>(WATTN_SMALL_ARGS);
    case 8: return launch_small_inst<false, false, 32, GATE>(WATTN_SMALL_ARGS);
    case 9: return launch_small_inst<false, true, 32, GATE>(WATTN_SMALL_ARGS);
    case 10: return launch_small_inst<true, false, 32, GATE>(WATTN_SMALL_ARGS);
    case 11: return launch_small_inst<true, true, 32, GATE>(WATTN_SMALL_ARGS);
    default: return hipErrorInvalidValue;
  }
#undef WATTN_SMALL_ARGS
}

template <int NW, bool GATE>
static hipError_t launch_bwd_nw(const WattnPlan& plan, bool rope, bool out_f32, int br, const void* q,
                                const void* k, const void* v, const void* out, const void* dout, const float* lse,
                                float* delta, float* dq, float* dk, float* dv, float* dtheta, const float* theta,
                                const void* bu, const void* bv, float* dbu, float* dbv, const void* gz, float* dz,
                                uint16_t* qt, uint16_t* dot, float* tmax, hipStream_t stream) {
#define WATTN_BWD_ARGS \
  plan, q, k, v, out, dout, lse, delta, dq, dk, dv, dtheta, theta, bu, bv, dbu, dbv, gz, dz, qt, dot, tmax, stream
  const int sel = (br / 16) * 4 + (rope ? 2 : 0) + (out_f32 ? 1 : 0);
  switch (sel) {
    case 0: return launch_bwd_inst<NW, false, false, 0, GATE>(WATTN_BWD_ARGS);
    case 1: return launch_bwd_inst<NW, false, true, 0, GATE>(WATTN_BWD_ARGS);
    case 2: return launch_bwd_inst<NW, true, false, 0, GATE>(WATTN_BWD_ARGS);
    case 3: return launch_bwd_inst<NW, true, true, 0, GATE>(WATTN_BWD_ARGS);
    case 4: return launch_bwd_inst<NW, false, false, 16, GATE>(WATTN_BWD_ARGS);
    case 5: return launch_bwd_inst<NW, false, true, 16, GATE>(WATTN_BWD_ARGS);
    case 6: return launch_bwd_inst<NW, true, false, 16, GATE>(WATTN_BWD_ARGS);
    case 7: return launch_bwd_inst<NW, true, true, 16, GATE>(WATTN_BWD_ARGS);
    case 8: return launch_bwd_inst<NW, false, false, 32, GATE>(WATTN_BWD_ARGS);
    case 9: return launch_bwd_inst<NW, false, true, 32, GATE>(WATTN_BWD_ARGS);
    case 10: return launch_bwd_inst<NW, true, false, 32, GATE>(WATTN_BWD_ARGS);
    case 11: return launch_bwd_inst<NW, true, true, 32, GATE>(WATTN_BWD_ARGS);
    default: return hipErrorInvalidValue;
  }
#undef WATTN_BWD_ARGS
}

hipError_t wattn_launch_bwd(const WattnPlan& plan, bool rope, bool out_f32, const void* q, const void* k,
                            const void* v, const void* out, const void* dout, const float* lse, float* scratch,
                            float* dq, float* dk, float* dv, float* dtheta, const float* theta, const void* bu,
                            const void* bv, int r, float* dbu, float* dbv, const void* gz, float* dz,
                            hipStream_t stream) {
  const int br = bu != nullptr ? r : 0;
  if (br != 0 && br != 16 && br != 32) return hipErrorInvalidValue;
  // scratch: delta [TH] floats, then (16-byte aligned) the fp16 q~ and bf16 dO~ rows [TH][32],
  // then one float per task (at most TH: every task holds at least one query row), the
  // largest output-gradient entry of the task's query tile, then the WATTN_DTHETA_COPIES
  // copies of the partial angle-gradient sums [copy][H][d/2]
  const int64_t th = (int64_t)plan.B * plan.Hg * plan.Wg * plan.H;
  if (plan.ntasks > th) return hipErrorInvalidValue;
  float* delta = scratch;
  uint16_t* qt = reinterpret_cast<uint16_t*>(scratch + ((th + 3) & ~int64_t(3)));
  uint16_t* dot = qt + th * D;
  float* tmax = reinterpret_cast<float*>(dot + th * D);
  float* dth_part = tmax + th;
  const int nth = plan.H * (D / 2);
  // one launch clears every atomic target: the angle-gradient copies and the bias-factor gradients
  const int64_t nb64 = (int64_t)plan.H * plan.M * plan.M * br;
  const int64_t nd64 = rope ? (int64_t)WATTN_DTHETA_COPIES * nth : 0;
  if (nb64 > 0x7fffff00LL || nd64 > 0x7fffff00LL) return hipErrorInvalidValue;  // one launch covers them
  const int nb = (int)nb64;
  const ZeroList z = {{dth_part, dbu, dbv}, {(int)nd64, nb, nb}};
  const int zmax = std::max(z.n[0], nb);
  if (zmax > 0) {
    hipLaunchKernelGGL(wattn_fill_zero_kernel, dim3((unsigned)((zmax + 255) / 256)), dim3(256), 0, stream, z);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool gate = gz != nullptr;
  hipError_t e;
  if (plan.nw == 2 && plan.M * plan.M <= SMALL_REGION) {
    // every region of a window of at most 8 x 8 fits one workgroup: one fused kernel
    e = gate ? launch_small<true>(plan, rope, out_f32, br, q, k, v, out, dout, lse, dq, dk, dv, dth_part, theta, bu,
                                  bv, dbu, dbv, gz, dz, stream)
             : launch_small<false>(plan, rope, out_f32, br, q, k, v, out, dout, lse, dq, dk, dv, dth_part, theta,
                                   bu, bv, dbu, dbv, gz, dz, stream);
  } else {
#define WATTN_BWD_ARGS plan, rope, out_f32, br, q, k, v, out, dout, lse, delta, dq, dk, dv, dth_part, theta, bu, bv, \
                       dbu, dbv, gz, dz, qt, dot, tmax, stream
    switch (plan.nw) {
      case 2: e = gate ? launch_bwd_nw<2, true>(WATTN_BWD_ARGS) : launch_bwd_nw<2, false>(WATTN_BWD_ARGS); break;
      case 4: e = gate ? launch_bwd_nw<4, true>(WATTN_BWD_ARGS) : launch_bwd_nw<4, false>(WATTN_BWD_ARGS); break;
      default: return hipErrorInvalidValue;
    }
#undef WATTN_BWD_ARGS
  }
  if (e != hipSuccess || !rope) return e;
  hipLaunchKernelGGL(wattn_dtheta_reduce_kernel, dim3((unsigned)nth), dim3(WATTN_DTHETA_COPIES), 0, stream,
                     static_cast<const float*>(dth_part), dtheta, nth);
  return hipGetLastError();
}
