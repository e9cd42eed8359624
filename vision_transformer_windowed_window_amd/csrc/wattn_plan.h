// wattn_plan.h -- launch plan shared by the host API and the kernels of libwattn.so.
//
// A shifted-window layer splits every window of the last row band and of the last column
// band into rectangular wrap regions (the tokens that stayed in place and the tokens that
// wrapped around from the other edge).  Tokens only attend within their region, so the
// bf16 path treats each region as an independent, unmasked attention problem; the masked
// pairs are never computed.  Windows that share a region shape form one segment.
//
// Task order (innermost first): query tile, head, window of the segment, image, segment.
// Segments are sorted by region size, largest first.
#pragma once

#include <stdint.h>

#define WATTN_MAX_SEG 9
#define WATTN_DTHETA_COPIES 256  // copies of the backward pass's partial angle-gradient sums
#define WATTN_F32_QTILE 256   // queries per workgroup of the fp32 path (one per thread)

// Divisors the kernel needs come with recip(d) = min(floor(2^32 / d), 2^32 - 1), computed on the
// host: the kernel then divides with a multiply-high and one correction step on the scalar
// unit (an integer division of uniform values would otherwise expand into a chain of vector
// reciprocal instructions).
struct WattnSeg {
  int wy0, nwy, wx0, nwx;  // windows of the segment: rows [wy0, wy0+nwy), cols [wx0, wx0+nwx)
  int r0, rh, c0, rw;      // region inside each window, window-local rows / cols
  int nqt;                 // query tiles per region
  int task_begin;          // index of the segment's first task
  uint32_t nqt_r, nwin_r, nwx_r;  // recip of nqt, nwy * nwx and nwx
  int step_i, step_j;      // key tile (16 nw keys) as region rows and columns: divmod(16 nw, rw)
  uint32_t rw_magic;       // multiplier of the per-lane index split by rw (0 for rw == 1)
};

struct WattnPlan {
  WattnSeg seg[WATTN_MAX_SEG];
  int nseg;
  int ntasks;
  int B, H, Hg, Wg, M, s;
  int nw;     // waves per workgroup of the bf16 path (2, 4 or 8); a task covers 32 nw queries
  int chunk;  // tasks kept together on one XCD (consecutive tasks share K/V in L2)
  int grid;   // launched workgroups: ntasks rounded up to a multiple of 8 * chunk
  uint32_t H_r, chunk_r;  // recip of H and of chunk
};

// floor(2^32 / d), clamped to 2^32 - 1 for d == 1 (d >= 1)
static inline uint32_t wattn_recip(uint32_t d) {
  return d <= 1 ? 0xffffffffu : (uint32_t)(0x100000000ULL / d);
}

// Plain per-window plan of the fp32 path: one workgroup per (query tile, head, window, image).
struct WattnF32Plan {
  int B, H, Hg, Wg, M, s;
  int nwx, nw, nqt;
  int grid;
};

