// wattn_api.cpp -- host side of libwattn.so: argument validation, launch planning and
// dispatch.  Every argument check runs before the first HIP call, so the error paths are
// testable on a machine without a GPU.

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "wattn.h"
#include "wattn_aux_plan.h"
#include "wattn_noalloc.h"
#include "wattn_plan.h"

hipError_t wattn_launch_bf16(const WattnPlan& plan, int nks, bool rope, bool out_f32, const void* q,
                             const void* k, const void* v, void* out, const float* theta, const void* bu,
                             const void* bv, float* lse, const void* gz, hipStream_t stream);
hipError_t wattn_launch_bwd(const WattnPlan& plan, bool rope, bool out_f32, const void* q, const void* k,
                            const void* v, const void* out, const void* dout, const float* lse, float* scratch,
                            float* dq, float* dk, float* dv, float* dtheta, const float* theta, const void* bu,
                            const void* bv, int r, float* dbu, float* dbv, const void* gz, float* dz,
                            hipStream_t stream);
hipError_t wattn_launch_select(const float* gate, int n, float tau, int* list, int* count, hipStream_t stream);
hipError_t wattn_launch_local(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v,
                              void* out, const int* list, const int* count, hipStream_t stream);
hipError_t wattn_launch_gated(const LocalPlan& P, bool out_f32, const void* q, const void* k, const void* v,
                              void* out, const float* gate, float tau, hipStream_t stream);
hipError_t wattn_launch_cla(const ClaPlan& P, const void* x, const float* w_dw, const float* b_dw, const float* w_pw,
                            const float* b_pw, void* z, hipStream_t stream);
hipError_t wattn_launch_linear(const LinearPlan& P, int act, bool res, bool out_f32, const void* x, const void* W,
                               const float* bias, const void* r, void* y, hipStream_t stream);
hipError_t wattn_launch_layernorm(const NormPlan& P, bool gather, const void* x, const float* gamma,
                                  const float* beta, void* y, hipStream_t stream);
hipError_t wattn_launch_stem(const StemPlan& P, const void* img, const void* W, const float* bias, void* y,
                             hipStream_t stream);
hipError_t wattn_launch_token_mean(const void* x, void* y, int B, int n, int C, hipStream_t stream);
hipError_t wattn_launch_f32(const WattnF32Plan& plan, int r, const void* q, const void* k, const void* v,
                            void* out, const float* theta, const void* bu, const void* bv, hipStream_t stream);

namespace {

constexpr int64_t kMaxElems = 1LL << 40;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_shape(int B, int H, int Hgrid, int Wgrid, int M, int shift) {
  if (B <= 0 || H <= 0 || Hgrid <= 0 || Wgrid <= 0 || M <= 0 || M > WATTN_MAX_M) return WATTN_ERR_SHAPE;
  if (Hgrid % M != 0 || Wgrid % M != 0) return WATTN_ERR_SHAPE;
  if (Hgrid > 65535 || Wgrid > 65535) return WATTN_ERR_SHAPE;
  if (shift < 0 || shift >= M) return WATTN_ERR_SHIFT;
  return WATTN_OK;
}

struct AxisSplit {
  // window groups along one axis: [w0, w0+nw) with region rows [r0, r0+rh)
  int n;
  int w0[3], nw[3], r0[3], rh[3];
};

AxisSplit split_axis(int G, int M, int s) {
  AxisSplit a{};
  const int nwin = G / M;
  if (s == 0) {
    a.n = 1;
    a.w0[0] = 0; a.nw[0] = nwin; a.r0[0] = 0; a.rh[0] = M;
    return a;
  }
  int n = 0;
  if (nwin > 1) {
    a.w0[n] = 0; a.nw[n] = nwin - 1; a.r0[n] = 0; a.rh[n] = M; ++n;
  }
  a.w0[n] = nwin - 1; a.nw[n] = 1; a.r0[n] = 0; a.rh[n] = M - s; ++n;   // tokens that stayed
  a.w0[n] = nwin - 1; a.nw[n] = 1; a.r0[n] = M - s; a.rh[n] = s; ++n;   // tokens that wrapped
  a.n = n;
  return a;
}

// Returns false if the task count would not fit the launch limits.
// Waves per workgroup of the bf16 path: wide workgroups amortise each staged K/V tile over
// more queries; narrow ones keep waves busy when windows (and their wrap regions) are small.
int waves_for_window(int M) { return M >= 24 ? 8 : (M >= 12 ? 4 : 2); }

bool build_plan(int B, int H, int Hg, int Wg, int M, int s, WattnPlan& P, int nw) {
  P = WattnPlan{};
  P.B = B; P.H = H; P.Hg = Hg; P.Wg = Wg; P.M = M; P.s = s;
  P.nw = nw;
  const int qtile = 32 * P.nw;
  const AxisSplit ay = split_axis(Hg, M, s), ax = split_axis(Wg, M, s);
  WattnSeg segs[WATTN_MAX_SEG];
  int ns = 0;
  for (int i = 0; i < ay.n; ++i)
    for (int j = 0; j < ax.n; ++j) {
      WattnSeg g{};
      g.wy0 = ay.w0[i]; g.nwy = ay.nw[i]; g.r0 = ay.r0[i]; g.rh = ay.rh[i];
      g.wx0 = ax.w0[j]; g.nwx = ax.nw[j]; g.c0 = ax.r0[j]; g.rw = ax.rh[j];
      g.nqt = (g.rh * g.rw + qtile - 1) / qtile;
      segs[ns++] = g;
    }
  std::stable_sort(segs, segs + ns, [](const WattnSeg& a, const WattnSeg& b) { return a.rh * a.rw > b.rh * b.rw; });
  int64_t begin = 0;
  const int ktile = 16 * P.nw;  // keys per LDS tile of the bf16 kernel
  for (int i = 0; i < ns; ++i) {
    WattnSeg& g = segs[i];
    g.task_begin = (int)begin;
    begin += (int64_t)g.nwy * g.nwx * g.nqt * H * B;
    if (begin > (1LL << 30)) return false;
    g.nqt_r = wattn_recip((uint32_t)g.nqt);
    g.nwin_r = wattn_recip((uint32_t)(g.nwy * g.nwx));
    g.nwx_r = wattn_recip((uint32_t)g.nwx);
    g.step_i = ktile / g.rw;
    g.step_j = ktile % g.rw;
    g.rw_magic = g.rw == 1 ? 0u : 0xffffffffu / (uint32_t)g.rw + 1u;
    P.seg[i] = g;
  }
  P.nseg = ns;
  P.ntasks = (int)begin;
  P.chunk = P.ntasks >= 128 ? 16 : std::max(1, (P.ntasks + 7) / 8);
  P.H_r = wattn_recip((uint32_t)H);
  P.chunk_r = wattn_recip((uint32_t)P.chunk);
  const int64_t unit = 8LL * P.chunk;
  P.grid = (int)(((int64_t)P.ntasks + unit - 1) / unit * unit);
  return true;
}

int pointer_ok(const void* p, size_t bytes) {
  if (p == nullptr) return WATTN_OK;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return WATTN_ERR_POINTER;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return WATTN_ERR_POINTER;
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return WATTN_ERR_POINTER;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), a = reinterpret_cast<uintptr_t>(p);
  if (a < b || a + bytes > b + size) return WATTN_ERR_POINTER;
  return WATTN_OK;
}

// Forward pass shared by wattn_forward, wattn_forward_lse and wattn_forward_gated (lse and the
// gate logits gz may be NULL).
int forward_impl(const void* q, const void* k, const void* v, void* out, float* lse, const void* gz, int B, int H,
                 int Hgrid, int Wgrid, int M, int shift, int d, const float* theta, const void* bias_u,
                 const void* bias_v, int r, int dtype, void* stream) {
  // ---- argument checks (no HIP call before this block ends)
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return WATTN_ERR_NULL;
  int st = check_shape(B, H, Hgrid, Wgrid, M, shift);
  if (st != WATTN_OK) return st;
  if (d != 32) return WATTN_ERR_HEAD_DIM;
  if (dtype != WATTN_BF16 && dtype != WATTN_FP32 && dtype != WATTN_BF16_OUT_FP32) return WATTN_ERR_DTYPE;
  if (r != 0 && r != 16 && r != 32) return WATTN_ERR_RANK;
  if (r == 0 && (bias_u != nullptr || bias_v != nullptr)) return WATTN_ERR_RANK;
  if (r > 0 && (bias_u == nullptr || bias_v == nullptr)) return WATTN_ERR_RANK;
  const int64_t elems = (int64_t)B * Hgrid * Wgrid * H * d;
  if (elems >= kMaxElems) return WATTN_ERR_SHAPE;
  if ((int64_t)Hgrid * Wgrid * H * d >= (1LL << 31)) return WATTN_ERR_SHAPE;  // 32-bit offsets within an image
  const size_t esz = (dtype == WATTN_FP32) ? 4 : 2;           // q, k, v, bias_u, bias_v
  const size_t osz = (dtype == WATTN_BF16) ? 2 : 4;           // out
  const size_t tbytes = (size_t)elems * esz;
  const size_t obytes = (size_t)elems * osz;
  const size_t th_bytes = (size_t)H * (d / 2) * sizeof(float);
  const size_t b_bytes = (size_t)H * M * M * r * esz;
  const Range ro{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + obytes};
  const Range ins[7] = {
      {reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + tbytes},
      {reinterpret_cast<uintptr_t>(k), reinterpret_cast<uintptr_t>(k) + tbytes},
      {reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(v) + tbytes},
      {reinterpret_cast<uintptr_t>(theta), reinterpret_cast<uintptr_t>(theta) + (theta ? th_bytes : 0)},
      {reinterpret_cast<uintptr_t>(bias_u), reinterpret_cast<uintptr_t>(bias_u) + (bias_u ? b_bytes : 0)},
      {reinterpret_cast<uintptr_t>(bias_v), reinterpret_cast<uintptr_t>(bias_v) + (bias_v ? b_bytes : 0)},
      {reinterpret_cast<uintptr_t>(gz), reinterpret_cast<uintptr_t>(gz) + (gz ? tbytes : 0)},
  };
  if (gz != nullptr && dtype == WATTN_FP32) return WATTN_ERR_DTYPE;
  for (const Range& x : ins)
    if (x.hi > x.lo && overlaps(ro, x)) return WATTN_ERR_ALIAS;
  const size_t lse_bytes = (size_t)(elems / d) * sizeof(float);
  if (lse != nullptr) {
    if (dtype == WATTN_FP32) return WATTN_ERR_DTYPE;
    const Range rl{reinterpret_cast<uintptr_t>(lse), reinterpret_cast<uintptr_t>(lse) + lse_bytes};
    if (overlaps(rl, ro)) return WATTN_ERR_ALIAS;
    for (const Range& x : ins)
      if (x.hi > x.lo && overlaps(rl, x)) return WATTN_ERR_ALIAS;
  }

  WattnPlan plan;
  WattnF32Plan fplan{};
  if (dtype != WATTN_FP32) {
    // With the rank-16 bias the 4-wave kernel fits four waves per SIMD (128 VGPRs) and the
    // 8-wave one runs a single workgroup per CU (it spills at 128): without RoPE the 4-wave
    // workgroups measured faster.  (The 4-wave RoPE table holds windows up to 26 wide, so the
    // bias with RoPE keeps the 8-wave kernel from M = 24 up.)
    const int nw = (r && theta == nullptr) ? std::min(waves_for_window(M), 4) : waves_for_window(M);
    if (!build_plan(B, H, Hgrid, Wgrid, M, shift, plan, nw)) return WATTN_ERR_SHAPE;
  } else {
    fplan.B = B; fplan.H = H; fplan.Hg = Hgrid; fplan.Wg = Wgrid; fplan.M = M; fplan.s = shift;
    fplan.nwx = Wgrid / M;
    fplan.nw = (Hgrid / M) * fplan.nwx;
    fplan.nqt = (M * M + WATTN_F32_QTILE - 1) / WATTN_F32_QTILE;
    const int64_t grid = (int64_t)fplan.nqt * H * fplan.nw * B;
    if (grid > (1LL << 30)) return WATTN_ERR_SHAPE;
    fplan.grid = (int)grid;
  }

  // ---- device checks
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  const void* ptrs[8] = {q, k, v, out, theta, bias_u, bias_v, gz};
  const size_t sizes[8] = {tbytes, tbytes, tbytes, obytes, th_bytes, b_bytes, b_bytes, tbytes};
  for (int i = 0; i < 8; ++i) {
    st = pointer_ok(ptrs[i], sizes[i]);
    if (st != WATTN_OK) return st;
  }
  if (lse != nullptr && (st = pointer_ok(lse, lse_bytes)) != WATTN_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype != WATTN_FP32)
    e = wattn_launch_bf16(plan, 2 + r / 16, theta != nullptr, dtype == WATTN_BF16_OUT_FP32, q, k, v, out, theta,
                          bias_u, bias_v, lse, gz, s);
  else
    e = wattn_launch_f32(fplan, r, q, k, v, out, theta, bias_u, bias_v, s);
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

}  // namespace

extern "C" int wattn_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int Hgrid,
                             int Wgrid, int M, int shift, int d, const float* theta, const void* bias_u,
                             const void* bias_v, int r, int dtype, void* stream) {
  return forward_impl(q, k, v, out, nullptr, nullptr, B, H, Hgrid, Wgrid, M, shift, d, theta, bias_u, bias_v, r,
                      dtype, stream);
}

extern "C" int wattn_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                                 int Hgrid, int Wgrid, int M, int shift, int d, const float* theta,
                                 const void* bias_u, const void* bias_v, int r, int dtype, void* stream) {
  if (lse == nullptr) return WATTN_ERR_NULL;
  return forward_impl(q, k, v, out, lse, nullptr, B, H, Hgrid, Wgrid, M, shift, d, theta, bias_u, bias_v, r, dtype,
                      stream);
}

extern "C" int wattn_forward_gated(const void* q, const void* k, const void* v, void* out, float* lse,
                                   const void* gate_z, int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                                   const float* theta, const void* bias_u, const void* bias_v, int r, int dtype,
                                   void* stream) {
  if (gate_z == nullptr) return WATTN_ERR_NULL;
  return forward_impl(q, k, v, out, lse, gate_z, B, H, Hgrid, Wgrid, M, shift, d, theta, bias_u, bias_v, r, dtype,
                      stream);
}

namespace {

// Backward scratch for `rows` query rows (T * H) and H heads: the rowsum statistic as float32
// [rows], padded to 16 bytes, then the rotated, scaled fp16 queries and the bf16 output
// gradient, [rows][32] each, then one float per task (a task holds at least one query row, so
// at most `rows`), then WATTN_DTHETA_COPIES copies of the partial angle-gradient sums [H][16].
int64_t backward_scratch_bytes(int64_t rows, int64_t H) {
  return (((rows + 3) & ~int64_t(3)) + 33 * rows + (int64_t)WATTN_DTHETA_COPIES * H * 16) * 4;
}

// Backward pass shared by wattn_backward, wattn_backward_gated (gz and dz both NULL or both
// set) and wattn_backward_noalloc (library_scratch: scratch is NULL on entry and the
// library-held array of wattn_noalloc.hip is used instead).
int backward_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  const void* gz, float* scratch, float* dq, float* dk, float* dv, float* dtheta, float* dz, int B,
                  int H, int Hgrid, int Wgrid, int M, int shift, int d, const float* theta, const void* bias_u,
                  const void* bias_v, int r, float* dbias_u, float* dbias_v, int dtype, void* stream,
                  bool library_scratch = false) {
  // ---- argument checks (no HIP call before this block ends)
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
      (scratch == nullptr && !library_scratch) || dq == nullptr || dk == nullptr || dv == nullptr)
    return WATTN_ERR_NULL;
  if ((theta == nullptr) != (dtheta == nullptr)) return WATTN_ERR_NULL;
  if ((gz == nullptr) != (dz == nullptr)) return WATTN_ERR_NULL;
  int st = check_shape(B, H, Hgrid, Wgrid, M, shift);
  if (st != WATTN_OK) return st;
  if (d != 32) return WATTN_ERR_HEAD_DIM;
  if (dtype != WATTN_BF16 && dtype != WATTN_BF16_OUT_FP32) return WATTN_ERR_DTYPE;
  if (r != 0 && r != 16 && r != 32) return WATTN_ERR_RANK;
  if (r == 0 && (bias_u != nullptr || bias_v != nullptr || dbias_u != nullptr || dbias_v != nullptr))
    return WATTN_ERR_RANK;
  if (r > 0 && (bias_u == nullptr || bias_v == nullptr || dbias_u == nullptr || dbias_v == nullptr))
    return WATTN_ERR_RANK;
  const int64_t elems = (int64_t)B * Hgrid * Wgrid * H * d;
  if (elems >= kMaxElems) return WATTN_ERR_SHAPE;
  if ((int64_t)Hgrid * Wgrid * H * d >= (1LL << 31)) return WATTN_ERR_SHAPE;
  const size_t tbytes = (size_t)elems * 2;                                    // q, k, v
  const size_t gbytes = (size_t)elems * (dtype == WATTN_BF16 ? 2 : 4);        // out, dout
  const size_t fbytes = (size_t)elems * 4;                                    // dq, dk, dv
  const size_t rbytes = (size_t)(elems / d) * 4;                              // lse
  const size_t sbytes = (size_t)backward_scratch_bytes(elems / d, H);         // scratch
  if (library_scratch && sbytes > (size_t)WATTN_NOALLOC_SCRATCH_BYTES) return WATTN_ERR_SCRATCH;
  const size_t th_bytes = (size_t)H * (d / 2) * sizeof(float);
  const size_t b_bytes = (size_t)H * M * M * r * 2;   // bias factors (bf16)
  const size_t db_bytes = (size_t)H * M * M * r * 4;  // their gradients (float32)
  auto rng = [](const void* p, size_t n) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (p ? n : 0)};
  };
  const Range ins[10] = {rng(q, tbytes), rng(k, tbytes), rng(v, tbytes), rng(out, gbytes), rng(dout, gbytes),
                         rng(lse, rbytes), rng(theta, th_bytes), rng(bias_u, b_bytes), rng(bias_v, b_bytes),
                         rng(gz, tbytes)};
  const Range outs[8] = {rng(scratch, sbytes), rng(dq, fbytes), rng(dk, fbytes), rng(dv, fbytes),
                         rng(dtheta, th_bytes), rng(dbias_u, db_bytes), rng(dbias_v, db_bytes), rng(dz, fbytes)};
  for (int i = 0; i < 8; ++i) {
    if (outs[i].hi == outs[i].lo) continue;
    for (const Range& x : ins)
      if (x.hi > x.lo && overlaps(outs[i], x)) return WATTN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (outs[j].hi > outs[j].lo && overlaps(outs[i], outs[j])) return WATTN_ERR_ALIAS;
  }
  if (reinterpret_cast<uintptr_t>(scratch) % 16 != 0) return WATTN_ERR_POINTER;
  WattnPlan plan;
  if (!build_plan(B, H, Hgrid, Wgrid, M, shift, plan, std::min(waves_for_window(M), 4))) return WATTN_ERR_SHAPE;

  // ---- device checks
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  const void* ptrs[18] = {q,     k,  v,      out,    dout,   lse,     scratch, dq, dk,
                          dv,    theta, dtheta, bias_u, bias_v, dbias_u, dbias_v, gz, dz};
  const size_t sizes[18] = {tbytes, tbytes, tbytes, gbytes, gbytes, rbytes, sbytes, fbytes, fbytes,
                            fbytes, th_bytes, th_bytes, b_bytes, b_bytes, db_bytes, db_bytes, tbytes, fbytes};
  for (int i = 0; i < 18; ++i) {
    st = pointer_ok(ptrs[i], sizes[i]);  // (a NULL library scratch is skipped)
    if (st != WATTN_OK) return st;
  }
  if (library_scratch) {
    void* p = nullptr;
    if (wattn_noalloc_scratch(static_cast<hipStream_t>(stream), &p) != hipSuccess) {
      (void)hipGetLastError();
      return WATTN_ERR_HIP;
    }
    scratch = static_cast<float*>(p);
  }
  const hipError_t e = wattn_launch_bwd(plan, theta != nullptr, dtype == WATTN_BF16_OUT_FP32, q, k, v, out, dout,
                                        lse, scratch, dq, dk, dv, dtheta, theta, bias_u, bias_v, r, dbias_u, dbias_v, gz,
                                        dz, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

}  // namespace

extern "C" int64_t wattn_backward_scratch_bytes(int B, int H, int Hgrid, int Wgrid, int d) {
  if (B <= 0 || H <= 0 || Hgrid <= 0 || Wgrid <= 0 || d != 32) return -1;
  return backward_scratch_bytes((int64_t)B * Hgrid * Wgrid * H, H);
}

extern "C" int wattn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, float* scratch, float* dq, float* dk, float* dv, float* dtheta, int B,
                              int H, int Hgrid, int Wgrid, int M, int shift, int d, const float* theta,
                              const void* bias_u, const void* bias_v, int r, float* dbias_u, float* dbias_v,
                              int dtype, void* stream) {
  return backward_impl(q, k, v, out, dout, lse, nullptr, scratch, dq, dk, dv, dtheta, nullptr, B, H, Hgrid, Wgrid, M,
                       shift, d, theta, bias_u, bias_v, r, dbias_u, dbias_v, dtype, stream);
}

extern "C" int wattn_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, float* dq, float* dk, float* dv,
                                      float* dtheta, int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                                      const float* theta, const void* bias_u, const void* bias_v, int r,
                                      float* dbias_u, float* dbias_v, int dtype, void* stream) {
  return backward_impl(q, k, v, out, dout, lse, nullptr, nullptr, dq, dk, dv, dtheta, nullptr, B, H, Hgrid, Wgrid,
                       M, shift, d, theta, bias_u, bias_v, r, dbias_u, dbias_v, dtype, stream, true);
}

extern "C" int wattn_backward_gated(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const float* lse, const void* gate_z, float* scratch, float* dq, float* dk,
                                    float* dv, float* dtheta, float* dgate_z, int B, int H, int Hgrid, int Wgrid,
                                    int M, int shift, int d, const float* theta, const void* bias_u,
                                    const void* bias_v, int r, float* dbias_u, float* dbias_v, int dtype,
                                    void* stream) {
  if (gate_z == nullptr || dgate_z == nullptr) return WATTN_ERR_NULL;
  return backward_impl(q, k, v, out, dout, lse, gate_z, scratch, dq, dk, dv, dtheta, dgate_z, B, H, Hgrid, Wgrid, M,
                       shift, d, theta, bias_u, bias_v, r, dbias_u, dbias_v, dtype, stream);
}

extern "C" int wattn_select_blocks(const float* gate, int nblocks, float tau, int* list, int* count, void* stream) {
  if (gate == nullptr || list == nullptr || count == nullptr) return WATTN_ERR_NULL;
  if (nblocks <= 0 || nblocks > WATTN_MAX_BLOCKS) return WATTN_ERR_SHAPE;
  const size_t gbytes = (size_t)nblocks * sizeof(float), lbytes = (size_t)nblocks * sizeof(int);
  auto rng = [](const void* p, size_t n) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n};
  };
  const Range rg = rng(gate, gbytes), rl = rng(list, lbytes), rc = rng(count, sizeof(int));
  if (overlaps(rl, rg) || overlaps(rc, rg) || overlaps(rc, rl)) return WATTN_ERR_ALIAS;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  int st;
  if ((st = pointer_ok(gate, gbytes)) != WATTN_OK || (st = pointer_ok(list, lbytes)) != WATTN_OK ||
      (st = pointer_ok(count, sizeof(int))) != WATTN_OK)
    return st;
  const hipError_t e = wattn_launch_select(gate, nblocks, tau, list, count, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

namespace {

// Checks and launch shared by the two forms of the residual correction: LISTED takes the block
// list of wattn_select_blocks, otherwise every block's workgroups route themselves by its gate.
int local_impl(const void* q, const void* k, const void* v, void* out, const int* list, const int* count,
               const float* gate, float tau, int B, int H, int Hgrid, int Wgrid, int w, int d, float eps, int dtype,
               void* stream, bool listed) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return WATTN_ERR_NULL;
  if (listed ? (list == nullptr || count == nullptr) : gate == nullptr) return WATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || Hgrid <= 0 || Wgrid <= 0 || Hgrid > 65535 || Wgrid > 65535) return WATTN_ERR_SHAPE;
  if (w != 4 && w != 8 && w != 12 && w != 16) return WATTN_ERR_SHAPE;
  if (Hgrid % w != 0 || Wgrid % w != 0) return WATTN_ERR_SHAPE;
  if (d != 32) return WATTN_ERR_HEAD_DIM;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return WATTN_ERR_VALUE;
  if (dtype != WATTN_BF16 && dtype != WATTN_BF16_OUT_FP32) return WATTN_ERR_DTYPE;
  const int64_t elems = (int64_t)B * Hgrid * Wgrid * H * d;
  if (elems >= kMaxElems || (int64_t)Hgrid * Wgrid * H * d >= (1LL << 31)) return WATTN_ERR_SHAPE;
  const int64_t nblocks = (int64_t)B * (Hgrid / w) * (Wgrid / w);
  if (nblocks > WATTN_MAX_BLOCKS || 8 * H * ((nblocks + 7) / 8) > 0x7fffffffLL) return WATTN_ERR_SHAPE;
  const size_t tbytes = (size_t)elems * 2, obytes = (size_t)elems * (dtype == WATTN_BF16 ? 2 : 4);
  const size_t lbytes = (size_t)nblocks * sizeof(int), gbytes = (size_t)nblocks * sizeof(float);
  auto rng = [](const void* p, size_t n) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (p ? n : 0)};
  };
  const Range ro = rng(out, obytes);
  const Range ins[6] = {rng(q, tbytes), rng(k, tbytes), rng(v, tbytes), rng(list, lbytes), rng(count, sizeof(int)),
                        rng(gate, gbytes)};
  for (const Range& x : ins)
    if (x.hi > x.lo && overlaps(ro, x)) return WATTN_ERR_ALIAS;

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  const void* ptrs[7] = {q, k, v, out, list, count, gate};
  const size_t sizes[7] = {tbytes, tbytes, tbytes, obytes, lbytes, sizeof(int), gbytes};
  for (int i = 0; i < 7; ++i) {
    const int st = pointer_ok(ptrs[i], sizes[i]);
    if (st != WATTN_OK) return st;
  }
  LocalPlan P;
  P.B = B; P.H = H; P.Hg = Hgrid; P.Wg = Wgrid; P.w = w;
  P.nWx = Wgrid / w;
  P.nW = (Hgrid / w) * P.nWx;
  P.nblocks = (int)nblocks;
  P.img_stride = (int64_t)Hgrid * Wgrid * H * d;
  P.eps = eps;
  const bool f32 = dtype == WATTN_BF16_OUT_FP32;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = listed ? wattn_launch_local(P, f32, q, k, v, out, list, count, s)
                              : wattn_launch_gated(P, f32, q, k, v, out, gate, tau, s);
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

}  // namespace

extern "C" int wattn_local_residual(const void* q, const void* k, const void* v, void* out, const int* list,
                                    const int* count, int B, int H, int Hgrid, int Wgrid, int w, int d, float eps,
                                    int dtype, void* stream) {
  return local_impl(q, k, v, out, list, count, nullptr, 0.f, B, H, Hgrid, Wgrid, w, d, eps, dtype, stream, true);
}

extern "C" int wattn_gated_local(const void* q, const void* k, const void* v, void* out, const float* gate,
                                 float tau, int B, int H, int Hgrid, int Wgrid, int w, int d, float eps, int dtype,
                                 void* stream) {
  return local_impl(q, k, v, out, nullptr, nullptr, gate, tau, B, H, Hgrid, Wgrid, w, d, eps, dtype, stream, false);
}

extern "C" int wattn_cla_logits(const void* x, const float* w_dw, const float* b_dw, const float* w_pw,
                                const float* b_pw, void* z, int B, int Hgrid, int Wgrid, int C, int dtype,
                                void* stream) {
  if (x == nullptr || w_dw == nullptr || w_pw == nullptr || z == nullptr) return WATTN_ERR_NULL;
  if (B <= 0 || Hgrid <= 0 || Wgrid <= 0 || Hgrid > 65535 || Wgrid > 65535) return WATTN_ERR_SHAPE;
  if (C < 32 || C > 256 || C % 32 != 0) return WATTN_ERR_HEAD_DIM;
  if (dtype != WATTN_BF16) return WATTN_ERR_DTYPE;
  const int64_t elems = (int64_t)B * Hgrid * Wgrid * C;
  if (elems >= kMaxElems || (int64_t)B * Hgrid * Wgrid >= (1LL << 31)) return WATTN_ERR_SHAPE;
  const size_t tbytes = (size_t)elems * 2, dw_bytes = (size_t)C * 9 * 4, pw_bytes = (size_t)C * C * 4,
               b_bytes = (size_t)C * 4;
  auto rng = [](const void* p, size_t n) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (p ? n : 0)};
  };
  const Range rz = rng(z, tbytes);
  const Range ins[5] = {rng(x, tbytes), rng(w_dw, dw_bytes), rng(b_dw, b_bytes), rng(w_pw, pw_bytes),
                        rng(b_pw, b_bytes)};
  for (const Range& r : ins)
    if (r.hi > r.lo && overlaps(rz, r)) return WATTN_ERR_ALIAS;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  const void* ptrs[6] = {x, w_dw, b_dw, w_pw, b_pw, z};
  const size_t sizes[6] = {tbytes, dw_bytes, b_bytes, pw_bytes, b_bytes, tbytes};
  for (int i = 0; i < 6; ++i) {
    const int st = pointer_ok(ptrs[i], sizes[i]);
    if (st != WATTN_OK) return st;
  }
  ClaPlan P;
  P.B = B; P.Hg = Hgrid; P.Wg = Wgrid; P.C = C;
  const int64_t rows = ((int64_t)Wgrid + 15) / 16 * Hgrid * B;  // at most the token count
  if (rows >= (1LL << 31)) return WATTN_ERR_SHAPE;
  P.rows = (int)rows;  // split into equal runs at launch
  P.per = P.grid = 0;
  const hipError_t e = wattn_launch_cla(P, x, w_dw, b_dw, w_pw, b_pw, z, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

// ---- model steps around the attention

namespace {

Range rng_of(const void* p, size_t n) {
  return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (p ? n : 0)};
}

bool any_overlap(Range out, const Range* ins, int n) {
  for (int i = 0; i < n; ++i)
    if (ins[i].hi > ins[i].lo && out.hi > out.lo && overlaps(out, ins[i])) return true;
  return false;
}

int device_ready() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return WATTN_ERR_HIP;
  }
  return WATTN_OK;
}

int pointers_ok(const void* const* ptrs, const size_t* sizes, int n) {
  for (int i = 0; i < n; ++i) {
    const int st = pointer_ok(ptrs[i], sizes[i]);
    if (st != WATTN_OK) return st;
  }
  return WATTN_OK;
}

int check_linear(int M, int N, int K, int split, int act, int dtype, bool res) {
  if (M <= 0 || N <= 0 || K <= 0 || M > (1 << 30) || N > (1 << 20) || K > (1 << 20)) return WATTN_ERR_SHAPE;
  if ((int64_t)((M + 127) / 128) * ((N + 127) / 128) > (1LL << 27)) return WATTN_ERR_SHAPE;  // grid size
  if (K % 32 != 0 || N % 4 != 0 || split <= 0 || split % 4 != 0 || N % split != 0) return WATTN_ERR_SHAPE;
  if (act != WATTN_ACT_NONE && act != WATTN_ACT_GELU) return WATTN_ERR_VALUE;
  if (dtype != WATTN_BF16 && dtype != WATTN_BF16_OUT_FP32) return WATTN_ERR_DTYPE;
  if (dtype == WATTN_BF16_OUT_FP32 && (act != WATTN_ACT_NONE || res)) return WATTN_ERR_DTYPE;
  return WATTN_OK;
}

LinearPlan linear_plan(int M, int N, int K, int split) {
  LinearPlan P;
  P.M = M; P.N = N; P.K = K; P.split = split;
  P.part_stride = (int64_t)M * split;
  return P;
}

}  // namespace

extern "C" int wattn_linear(const void* x, const void* W, const float* bias, const void* residual, void* y, int M,
                            int N, int K, int split, int act, int dtype, void* stream) {
  if (x == nullptr || W == nullptr || y == nullptr) return WATTN_ERR_NULL;
  int st = check_linear(M, N, K, split, act, dtype, residual != nullptr);
  if (st != WATTN_OK) return st;
  const size_t xb = (size_t)M * K * 2, wb = (size_t)N * K * 2, bb = (size_t)N * 4, rb = (size_t)M * N * 2;
  const size_t yb = (size_t)M * N * (dtype == WATTN_BF16 ? 2 : 4);
  const Range ins[3] = {rng_of(x, xb), rng_of(W, wb), rng_of(bias, bb)};
  if (any_overlap(rng_of(y, yb), ins, 3)) return WATTN_ERR_ALIAS;
  if (residual != nullptr && residual != y && overlaps(rng_of(y, yb), rng_of(residual, rb))) return WATTN_ERR_ALIAS;
  if ((st = device_ready()) != WATTN_OK) return st;
  const void* ptrs[5] = {x, W, bias, residual, y};
  const size_t sizes[5] = {xb, wb, bb, rb, yb};
  if ((st = pointers_ok(ptrs, sizes, 5)) != WATTN_OK) return st;
  const hipError_t e = wattn_launch_linear(linear_plan(M, N, K, split), act, residual != nullptr,
                                           dtype == WATTN_BF16_OUT_FP32, x, W, bias, residual, y,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

namespace {

int norm_impl(const void* x, const float* gamma, const float* beta, void* y, int64_t T, int C, int Hg, int Wg,
              float eps, bool gather, void* stream) {
  if (x == nullptr || gamma == nullptr || beta == nullptr || y == nullptr) return WATTN_ERR_NULL;
  if (T <= 0 || C <= 0 || C % 8 != 0 || C > (1 << 16) || T > (1LL << 31)) return WATTN_ERR_SHAPE;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return WATTN_ERR_VALUE;
  const int Ct = gather ? 4 * C : C;
  const int64_t in_tokens = gather ? 4 * T : T;
  const size_t xb = (size_t)in_tokens * C * 2, yb = (size_t)T * Ct * 2, gb = (size_t)Ct * 4;
  const Range ins[3] = {rng_of(x, xb), rng_of(gamma, gb), rng_of(beta, gb)};
  if (any_overlap(rng_of(y, yb), ins, 3)) return WATTN_ERR_ALIAS;
  int st;
  if ((st = device_ready()) != WATTN_OK) return st;
  const void* ptrs[4] = {x, gamma, beta, y};
  const size_t sizes[4] = {xb, gb, gb, yb};
  if ((st = pointers_ok(ptrs, sizes, 4)) != WATTN_OK) return st;
  NormPlan P;
  P.T = T; P.C = C; P.Hg = Hg; P.Wg = Wg; P.eps = eps;
  const hipError_t e = wattn_launch_layernorm(P, gather, x, gamma, beta, y, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

}  // namespace

extern "C" int wattn_layernorm(const void* x, const float* gamma, const float* beta, void* y, int64_t T, int C,
                               float eps, void* stream) {
  return norm_impl(x, gamma, beta, y, T, C, 0, 0, eps, false, stream);
}

extern "C" int wattn_patch_merge_norm(const void* x, const float* gamma, const float* beta, void* y, int B,
                                      int Hgrid, int Wgrid, int C, float eps, void* stream) {
  if (B <= 0 || Hgrid <= 0 || Wgrid <= 0 || Hgrid % 2 != 0 || Wgrid % 2 != 0 || Hgrid > 65535 || Wgrid > 65535)
    return WATTN_ERR_SHAPE;
  return norm_impl(x, gamma, beta, y, (int64_t)B * (Hgrid / 2) * (Wgrid / 2), C, Hgrid, Wgrid, eps, true, stream);
}

extern "C" int wattn_stem_conv(const void* img, const void* W, const float* bias, void* y, int B, int Himg, int Wimg,
                               int Cin, int Cout, int p, void* stream) {
  if (img == nullptr || W == nullptr || bias == nullptr || y == nullptr) return WATTN_ERR_NULL;
  if (B <= 0 || Himg <= 0 || Wimg <= 0 || Cin <= 0 || Cout <= 0 || p <= 0 || Cout % 32 != 0) return WATTN_ERR_SHAPE;
  if (Himg % p != 0 || Wimg % p != 0 || Himg > 65535 || Wimg > 65535) return WATTN_ERR_SHAPE;
  const int k = 2 * p - 1;
  if ((int64_t)k * k * Cin * Cout * 4 > 65536) return WATTN_ERR_SHAPE;  // weights staged in 64 KB of LDS
  const int Ho = Himg / p, Wo = Wimg / p;
  if ((int64_t)B * Ho * Wo * (Cout / 32) >= (1LL << 31)) return WATTN_ERR_SHAPE;
  const size_t ib = (size_t)B * Himg * Wimg * Cin * 2, wb = (size_t)Cout * Cin * k * k * 2, bb = (size_t)Cout * 4;
  const size_t yb = (size_t)B * Ho * Wo * Cout * 2;
  const Range ins[3] = {rng_of(img, ib), rng_of(W, wb), rng_of(bias, bb)};
  if (any_overlap(rng_of(y, yb), ins, 3)) return WATTN_ERR_ALIAS;
  int st;
  if ((st = device_ready()) != WATTN_OK) return st;
  const void* ptrs[4] = {img, W, bias, y};
  const size_t sizes[4] = {ib, wb, bb, yb};
  if ((st = pointers_ok(ptrs, sizes, 4)) != WATTN_OK) return st;
  StemPlan P;
  P.B = B; P.Hi = Himg; P.Wi = Wimg; P.Cin = Cin; P.Cout = Cout; P.p = p; P.Ho = Ho; P.Wo = Wo;
  const hipError_t e = wattn_launch_stem(P, img, W, bias, y, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

extern "C" int wattn_token_mean(const void* x, void* y, int B, int n, int C, void* stream) {
  if (x == nullptr || y == nullptr) return WATTN_ERR_NULL;
  if (B <= 0 || n <= 0 || C <= 0 || C % 8 != 0 || B > 65535 || (int64_t)B * C >= (1LL << 31) ||
      (int64_t)B * n * C >= kMaxElems)
    return WATTN_ERR_SHAPE;
  const size_t xb = (size_t)B * n * C * 2, yb = (size_t)B * C * 2;
  if (overlaps(rng_of(y, yb), rng_of(x, xb))) return WATTN_ERR_ALIAS;
  int st;
  if ((st = device_ready()) != WATTN_OK) return st;
  const void* ptrs[2] = {x, y};
  const size_t sizes[2] = {xb, yb};
  if ((st = pointers_ok(ptrs, sizes, 2)) != WATTN_OK) return st;
  const hipError_t e = wattn_launch_token_mean(x, y, B, n, C, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WATTN_OK : WATTN_ERR_HIP;
}

extern "C" int64_t wattn_swin_block_workspace(int B, int Hgrid, int Wgrid, int C) {
  if (B <= 0 || Hgrid <= 0 || Wgrid <= 0 || C <= 0) return -1;
  return (int64_t)B * Hgrid * Wgrid * C * 2 * 5;  // normalised x, q/k/v (the attention output reuses the first)
}

extern "C" int wattn_swin_block(void* x, const wattn_block_params_t* p, void* workspace, int64_t workspace_bytes,
                                int B, int Hgrid, int Wgrid, int C, int H, int M, int shift, void* stream) {
  if (x == nullptr || p == nullptr || workspace == nullptr) return WATTN_ERR_NULL;
  if (p->ln1_g == nullptr || p->ln1_b == nullptr || p->w_qkv == nullptr || p->w_proj == nullptr ||
      p->ln2_g == nullptr || p->ln2_b == nullptr || p->w_fc1 == nullptr || p->w_fc2 == nullptr)
    return WATTN_ERR_NULL;
  int st = check_shape(B, H, Hgrid, Wgrid, M, shift);
  if (st != WATTN_OK) return st;
  if (C <= 0 || C % H != 0 || C / H != 32 || C % 32 != 0) return WATTN_ERR_HEAD_DIM;
  const int64_t T = (int64_t)B * Hgrid * Wgrid;
  if (T * C * 4 >= kMaxElems || (int64_t)Hgrid * Wgrid * C >= (1LL << 31) || T >= (1LL << 30)) return WATTN_ERR_SHAPE;
  if (workspace_bytes < wattn_swin_block_workspace(B, Hgrid, Wgrid, C)) return WATTN_ERR_SHAPE;
  const size_t xb = (size_t)T * C * 2;
  if (overlaps(rng_of(x, xb), rng_of(workspace, (size_t)workspace_bytes))) return WATTN_ERR_ALIAS;
  WattnPlan plan;
  if (!build_plan(B, H, Hgrid, Wgrid, M, shift, plan, waves_for_window(M))) return WATTN_ERR_SHAPE;
  if ((st = device_ready()) != WATTN_OK) return st;
  const size_t cb = (size_t)C * 4;
  const void* ptrs[16] = {x, workspace, p->ln1_g, p->ln1_b, p->w_qkv, p->b_qkv, p->w_proj, p->b_proj,
                          p->ln2_g, p->ln2_b, p->w_fc1, p->b_fc1, p->w_fc2, p->b_fc2, p->theta, nullptr};
  const size_t sizes[16] = {xb, (size_t)workspace_bytes, cb, cb, (size_t)3 * C * C * 2, 3 * cb,
                            (size_t)C * C * 2, cb, cb, cb, (size_t)4 * C * C * 2, 4 * cb, (size_t)4 * C * C * 2, cb,
                            (size_t)H * 16 * 4, 0};
  if ((st = pointers_ok(ptrs, sizes, 15)) != WATTN_OK) return st;

  // workspace: h = [0, TC) (normalised x, then the attention output, then the second norm),
  // q/k/v = [TC, 4TC), MLP hidden = [TC, 5TC)
  uint16_t* ws = static_cast<uint16_t*>(workspace);
  uint16_t* h = ws;
  uint16_t* qkv = ws + T * C;
  uint16_t* hid = ws + T * C;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  NormPlan np;
  np.T = T; np.C = C; np.Hg = 0; np.Wg = 0; np.eps = 1e-5f;
  hipError_t e;
  if ((e = wattn_launch_layernorm(np, false, x, p->ln1_g, p->ln1_b, h, s)) != hipSuccess) return WATTN_ERR_HIP;
  if ((e = wattn_launch_linear(linear_plan((int)T, 3 * C, C, C), WATTN_ACT_NONE, false, false, h, p->w_qkv, p->b_qkv,
                               nullptr, qkv, s)) != hipSuccess)
    return WATTN_ERR_HIP;
  if ((e = wattn_launch_bf16(plan, 2, p->theta != nullptr, false, qkv, qkv + T * C, qkv + 2 * T * C, h, p->theta,
                             nullptr, nullptr, nullptr, nullptr, s)) != hipSuccess)
    return WATTN_ERR_HIP;
  if ((e = wattn_launch_linear(linear_plan((int)T, C, C, C), WATTN_ACT_NONE, true, false, h, p->w_proj, p->b_proj, x,
                               x, s)) != hipSuccess)
    return WATTN_ERR_HIP;
  if ((e = wattn_launch_layernorm(np, false, x, p->ln2_g, p->ln2_b, h, s)) != hipSuccess) return WATTN_ERR_HIP;
  if ((e = wattn_launch_linear(linear_plan((int)T, 4 * C, C, 4 * C), WATTN_ACT_GELU, false, false, h, p->w_fc1,
                               p->b_fc1, nullptr, hid, s)) != hipSuccess)
    return WATTN_ERR_HIP;
  if ((e = wattn_launch_linear(linear_plan((int)T, C, 4 * C, C), WATTN_ACT_NONE, true, false, hid, p->w_fc2, p->b_fc2,
                               x, x, s)) != hipSuccess)
    return WATTN_ERR_HIP;
  return WATTN_OK;
}

extern "C" int64_t wattn_pair_count(int B, int H, int Hgrid, int Wgrid, int M, int shift) {
  if (check_shape(B, H, Hgrid, Wgrid, M, shift) != WATTN_OK) return -1;
  const AxisSplit ay = split_axis(Hgrid, M, shift), ax = split_axis(Wgrid, M, shift);
  int64_t total = 0;
  for (int i = 0; i < ay.n; ++i)
    for (int j = 0; j < ax.n; ++j) {
      const int64_t ntok = (int64_t)ay.rh[i] * ax.rh[j];
      total += (int64_t)ay.nw[i] * ax.nw[j] * ntok * ntok;
    }
  return total * B * H;
}

extern "C" const char* wattn_status_string(int status) {
  switch (status) {
    case WATTN_OK: return "ok";
    case WATTN_ERR_NULL: return "null q, k, v or out pointer";
    case WATTN_ERR_SHAPE: return "invalid or unsupported sizes (B, H, grid, M)";
    case WATTN_ERR_SHIFT: return "shift outside [0, M)";
    case WATTN_ERR_HEAD_DIM: return "unsupported head dimension (supported: 32)";
    case WATTN_ERR_RANK: return "unsupported bias rank or bias pointers inconsistent with r";
    case WATTN_ERR_DTYPE: return "unknown dtype";
    case WATTN_ERR_ALIAS: return "out overlaps an input buffer";
    case WATTN_ERR_HIP: return "HIP runtime error (no device or launch failure)";
    case WATTN_ERR_POINTER: return "buffer is not device-accessible memory of the required size";
    case WATTN_ERR_VALUE: return "scalar parameter out of range (eps must be finite and >= 0)";
    case WATTN_ERR_SCRATCH: return "problem needs more scratch than the library holds (wattn_backward_noalloc)";
    default: return "unknown status";
  }
}

extern "C" int wattn_abi_version(void) { return WATTN_ABI_VERSION; }
