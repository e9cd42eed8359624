// wattn_aux_plan.h -- launch descriptions of the kernels beside the window attention: the gated
// local path, the gate-logit convolutions and the model steps (linear layers, norms, stem).
// Shared by the host code and the device code of those kernels.

#pragma once

#include <stdint.h>

// Launch description of the gated local path: the w x w block grid of the token grid.
// Block index = b * nW + wy * nWx + wx (nW = nWy * nWx blocks per image).
struct LocalPlan {
  int B, H, Hg, Wg, w;
  int nWx, nW, nblocks;
  int64_t img_stride;  // elements of one image: Hg * Wg * H * d
  float eps;           // denominator guard of the linear attention
};

// Launch description of the gate-logit convolutions: the token grid, the channel count and the
// number of workgroups (one per strip of 16 columns and 16 rows of an image).
struct ClaPlan {
  int B, Hg, Wg, C;
  int rows;  // output rows of all 16-column strips: B * ceil(Wg / 16) * Hg
  int per;   // rows per workgroup (set at launch)
  int grid;  // workgroups (set at launch)
};

// Linear layer y = act(x W^T + b) (+ res): x [M][K], W [N][K]; output column n is stored in
// part n / split at part * part_stride + m * split + n % split.
struct LinearPlan {
  int M, N, K, split;
  int64_t part_stride;
};

// Layer norm over C channels of T output tokens (gathered 2 x 2 from a Hg x Wg map for patch
// merging, in which case the row has 4C channels).
struct NormPlan {
  int64_t T;
  int C, Hg, Wg;
  float eps;
};

// Overlapping stem: kernel 2p - 1, stride p, padding p - 1, on an NHWC image.
struct StemPlan {
  int B, Hi, Wi, Cin, Cout, p, Ho, Wo;
};
