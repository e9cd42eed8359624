/*
 * wattn.h -- C ABI of libwattn.so: fused shifted-window softmax attention with
 * window-local learned 2D RoPE and a folded low-rank position bias, for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *
 *   FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with
 *   Memory Efficient Attention -- "What it is": attention is restricted to non-overlapping
 *   M x M windows of the token grid.  "How it works", first change: the window attention
 *   is one IO-aware fused pass with an online softmax; the N x N score matrix (N = M*M)
 *   is never stored and the result is exact softmax attention.  Second change: Q and K
 *   get a window-local learned 2D rotary embedding (first half of the head dimension
 *   encodes the row y, second half the column x, theta = exp(omega)); in shifted-window
 *   layers the grid is cyclically shifted, coordinates are recomputed per window, and the
 *   wrapped windows are masked.  Mixed-precision note (closing developer paragraph):
 *   bf16 Q/K/V, RoPE applied in fp32, softmax accumulated in fp32.
 *
 *   Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution Transformer with
 *   FlashAttention -- section 2.1: a low-rank bias enters as extra channels,
 *   [Q_c, Q_p][K_c, K_p]^T = Q_c K_c^T + Q_p K_p^T, so no N x N bias matrix exists.
 *
 * For image b, head h and window w of the grid rolled by -shift, with window-local
 * coordinates p_n = (r_n, c_n) in [0, M)^2 (n = r*M + c):
 *
 *   logit[n][m] = <R(p_n) q_n, R(p_m) k_m> / sqrt(d)  +  <bias_u[h][n], bias_v[h][m]>
 *                 + (0 if n and m lie in the same wrap region of the window, else -inf)
 *   out_n       = sum_m softmax_m(logit[n][.]) v_m
 *
 * q_n is read from, and out_n written to, the token's ORIGINAL grid position
 * ((Y + shift) mod Hgrid, (X + shift) mod Wgrid) where (Y, X) is its rolled position, so
 * the cyclic shift and its reversal are part of the call.  R(p) rotates adjacent pairs
 * (2j, 2j+1) counter-clockwise by r*theta[h][j] for j < d/4 and by c*theta[h][j] for
 * j >= d/4.  Region labels per axis (rolled coordinate P on an axis of length G):
 * 0 if P < G - M, 1 if P < G - shift, else 2; a pair is masked iff the labels differ on
 * either axis (no pair is masked when shift == 0).
 */
#ifndef WATTN_H
#define WATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WATTN_ABI_VERSION 5

/* Element types.  The bf16 modes take bf16 q, k, v and run both products on the matrix
 * cores with fp32 RoPE, fp32 softmax and fp32 accumulation: QK^T on fp16 operands (the
 * rotated q and k rounded once to fp16, see wattn_forward) and PV on bf16 operands.  They
 * differ only in the type of `out`.  A bf16 `out` adds its own rounding (up to 2^-9
 * relative) on top of the kernel's error. */
typedef enum {
  WATTN_BF16 = 0,          /* q, k, v, bias_u, bias_v and out in bfloat16 */
  WATTN_FP32 = 1,          /* everything in float32 (plain fp32 arithmetic, no matrix cores) */
  WATTN_BF16_OUT_FP32 = 2  /* q, k, v, bias_u, bias_v in bfloat16, out in float32 */
} wattn_dtype_t;

/* Status codes.  Every invalid argument is detected on the host before any HIP call,
 * and nothing is written when a call fails. */
typedef enum {
  WATTN_OK = 0,
  WATTN_ERR_NULL = 1,     /* q, k, v or out is NULL */
  WATTN_ERR_SHAPE = 2,    /* a size <= 0, M > WATTN_MAX_M, grid not a multiple of M, a grid side
                             above 65535, or one image holding 2^31 or more elements */
  WATTN_ERR_SHIFT = 3,    /* shift outside [0, M) */
  WATTN_ERR_HEAD_DIM = 4, /* d not supported (this version: d == 32) */
  WATTN_ERR_RANK = 5,     /* r not in {0, 16}, or bias pointers inconsistent with r */
  WATTN_ERR_DTYPE = 6,    /* unknown dtype enum */
  WATTN_ERR_ALIAS = 7,    /* out overlaps an input buffer */
  WATTN_ERR_HIP = 8,      /* HIP runtime error (no device, launch failure, ...) */
  WATTN_ERR_POINTER = 9,  /* a buffer is not device-accessible memory */
  WATTN_ERR_VALUE = 10,   /* a scalar parameter out of range (eps of the gated local path) */
  WATTN_ERR_SCRATCH = 11  /* the call needs more scratch than wattn_backward_noalloc holds */
} wattn_status_t;

#define WATTN_MAX_M 128
#define WATTN_MAX_BLOCKS (1 << 22) /* blocks of one gated-local-path call */

/*
 * wattn_forward -- out = shifted-window attention of (q, k, v); see the header comment.
 *
 * q, k, v, out : device pointers, [B][Hgrid][Wgrid][H][d] contiguous (token-major, the
 *                layout a qkv projection writes), element types given by `dtype`.
 *                Read-only except `out`.  `out` must not overlap any input.
 * B, H         : images and heads, >= 1.
 * Hgrid, Wgrid : token grid; each a positive multiple of M.
 * M            : window side, 1 <= M <= WATTN_MAX_M (N = M*M tokens per window).
 * shift        : cyclic shift in [0, M); 0 = regular windows.
 * d            : head dimension (supported: 32).
 * theta        : device pointer, float32 [H][d/2] rotation-pair frequencies
 *                (theta = exp(omega)), or NULL for no rotary embedding.
 * bias_u,
 * bias_v       : device pointers, [H][M*M][r] of q's element type, indexed by the
 *                window-local token index n = r*M + c; both NULL when r == 0.
 * r            : bias rank, 0, 16 or 32 (d + r a multiple of 16 that one or two k = 32
 *                matrix-core products carry: a rank-16 bias is zero-padded to the second
 *                product, which on this GPU costs the same as a k = 16 product, and a
 *                rank-32 bias fills it).
 * dtype        : a wattn_dtype_t value.
 * stream       : hipStream_t to launch on; NULL = the default stream.
 *
 * The call only launches work: it returns after enqueueing on `stream`, allocates no
 * memory, keeps no state and is safe to call from several threads.  The caller owns
 * every buffer and must keep it alive until the stream has run the work.  Scale is
 * d^-1/2 on the content logits; the bias is added unscaled.  NaN or Inf inputs
 * propagate to the output and are not checked.
 *
 * bf16 modes: after the fp32 rotation, q * log2(e) / sqrt(d), k and the bias factors
 * (u * log2(e), v) are rounded once to fp16 for the score product on the matrix cores
 * (fp16 keeps three more significand bits than bf16); P is rounded to bf16 for the
 * value product.  fp16 holds magnitudes below 65504, so q entries must stay below about
 * 1.8e5 and k and bias-factor entries below about 4.6e4 (a rotation can grow a
 * component by sqrt(2)); larger entries overflow and give non-finite outputs.
 *
 * Returns WATTN_OK or one of the WATTN_ERR_* codes above.
 */
int wattn_forward(const void* q, const void* k, const void* v, void* out,
                  int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                  const float* theta, const void* bias_u, const void* bias_v, int r,
                  int dtype, void* stream);

/*
 * wattn_forward_lse -- wattn_forward that also stores the row statistic the backward pass
 * needs: lse[b][y][x][h] = log sum_m exp(logit[n][m]) (natural log, over the keys the query
 * sees) for the query token stored at original position (y, x).
 *
 * lse : float32 device pointer, [B][Hgrid][Wgrid][H], written (caller-owned).  It must not
 *       overlap any other argument buffer (WATTN_ERR_ALIAS); NULL gives WATTN_ERR_NULL.
 * dtype must be WATTN_BF16 or WATTN_BF16_OUT_FP32 (WATTN_ERR_DTYPE otherwise).  All other
 * arguments, checks and numerics are those of wattn_forward.
 *
 * The row statistic is the softmax normaliser of the FLASHSWIN page's fused kernel ("How it
 * works", first change: online softmax per tile); keeping it makes the backward pass an
 * exact recomputation of the same softmax.
 */
int wattn_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                      const float* theta, const void* bias_u, const void* bias_v, int r,
                      int dtype, void* stream);

/*
 * wattn_backward_scratch_bytes -- bytes of the scratch buffer wattn_backward and
 * wattn_backward_gated take for these sizes: 4 * (ceil4(T) + 33 T + 4096 H) with T = B Hgrid
 * Wgrid H query rows (4096 H: 256 copies of the partial angle-gradient sums).  -1 for a size
 * <= 0 or d != 32.
 */
int64_t wattn_backward_scratch_bytes(int B, int H, int Hgrid, int Wgrid, int d);

/*
 * wattn_backward -- gradients of loss = sum(dout * out) of the shifted-window attention
 * (the FLASHSWIN page's memory claims cover the scores and their gradient: the backward
 * pass recomputes P per tile from q, k and lse and never stores an N x N matrix).
 *
 * Inputs (device pointers, caller-owned, read only):
 *   q, k, v : bfloat16 [B][Hgrid][Wgrid][H][d], the forward pass's inputs.
 *   out     : the forward pass's output, dout: the gradient of the loss with respect to it;
 *             both [B][Hgrid][Wgrid][H][d], bfloat16 for dtype WATTN_BF16 and float32 for
 *             WATTN_BF16_OUT_FP32.
 *   lse     : float32 [B][Hgrid][Wgrid][H] from wattn_forward_lse on the same inputs.
 *   theta   : float32 [H][d/2] as in the forward pass, or NULL (no RoPE).
 * Outputs (device pointers, caller-owned, overwritten):
 *   scratch : wattn_backward_scratch_bytes(B, H, Hgrid, Wgrid, d) bytes of device memory,
 *             16-byte aligned (WATTN_ERR_POINTER otherwise), contents undefined on entry and
 *             on return.  The query-tile kernel writes rowsum(dout * out) per query, the
 *             rotated and scaled queries (fp16), the output gradient (bf16) and the largest
 *             output-gradient entry of each query tile there once; the key-tile kernel
 *             streams them back instead of redoing that work per tile.  Every kernel adds its
 *             angle-gradient sums into the copies at the end of the scratch.
 *   dq, dk, dv : float32 [B][Hgrid][Wgrid][H][d].
 *   dtheta  : float32 [H][d/2], written by a last small kernel from partial sums that the
 *             waves add into 256 copies in the scratch with atomic adds, so its last bits
 *             depend on the order of the additions; required iff theta is not NULL.
 *   dbias_u, dbias_v : float32 [H][M*M][r], the gradients of the bias factors (summed over
 *             every window and image, which share them; zeroed, then accumulated with atomic
 *             adds); required iff r > 0.
 * bias_u, bias_v, r : the forward pass's bias factors (bfloat16 [H][M*M][r]) and rank, as in
 *             wattn_forward: NULL, NULL, 0 or both set with r == 16 or r == 32
 *             (WATTN_ERR_RANK otherwise, also when the dbias pointers do not match).
 * Sizes, shift and d follow wattn_forward.  No output may overlap an input or another
 * output (WATTN_ERR_ALIAS).  Asynchronous on `stream`: one fill launch for the accumulated
 * outputs, then for M <= 8 one fused kernel (a workgroup holds a whole wrap region), for
 * larger windows two (one per query tile: delta, dq, the q part of dtheta, dbias_u; one per
 * key tile: dk, dv, the k part of dtheta, dbias_v), and with theta the kernel that sums the
 * angle-gradient copies into dtheta.
 *
 * Numerics: the scores are recomputed as in the forward pass (fp16 operands, P =
 * exp2(s log2(e) - lse log2(e)) in fp32); P is rounded to bf16 for dv, dS = P (dP - delta)
 * to fp16 for dq and dk; everything accumulates in fp32.  dS is rounded with a power-of-two
 * scale 2^e that puts the largest output-gradient entry in [4, 8) (per query row for dq and
 * dbias_u, per wrap region -- the queries a key attends with -- for dk, dv and dbias_v;
 * |e| <= 96), and the fp32 products are divided by 2^e, so the relative accuracy of every
 * gradient does not depend on the magnitude of dout, also where it differs between regions
 * (gradients scale exactly with a power-of-two factor on dout).  No atomic operation takes
 * part in dq, dk or dv, so they are bitwise reproducible.
 */
int wattn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, float* scratch, float* dq, float* dk, float* dv, float* dtheta,
                   int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                   const float* theta, const void* bias_u, const void* bias_v, int r,
                   float* dbias_u, float* dbias_v, int dtype, void* stream);

/*
 * wattn_backward_noalloc -- wattn_backward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without `scratch`, the same kernels, outputs and numerics.
 *
 * The scratch comes from a file-scope device array of the library (64 MiB on every GPU the
 * library runs on, held until the process ends), so the call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.  Calls that need more than that, i.e. more than
 * about 493300 query rows B * Hgrid * Wgrid * H (wattn_backward_scratch_bytes > 64 MiB), return
 * WATTN_ERR_SCRATCH before any HIP call.  The first call on a device looks the array's address
 * up on that device (the device of `stream`; the current one for the null stream).
 *
 * Every call on one GPU shares that GPU's array and leaves its contents behind; what must
 * start at zero is cleared by the call itself on `stream`.  Calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race on the array and
 * give undefined results: order them on one stream.
 */
int wattn_backward_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                           const float* lse, float* dq, float* dk, float* dv, float* dtheta,
                           int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                           const float* theta, const void* bias_u, const void* bias_v, int r,
                           float* dbias_u, float* dbias_v, int dtype, void* stream);

/*
 * Convolutional gate on the attention output (Rank-Factorized Implicit Neural Bias: Scaling
 * Super-Resolution Transformer with FlashAttention, section 2.2): a 3x3 depth-wise and a 1x1
 * point-wise convolution of the layer input give gate logits z, a sigmoid turns them into a
 * gating map, and the map multiplies the attention output channel by channel:
 *
 *   out[b][y][x][h][j] = sigmoid(z[b][y][x][h][j]) * attention[b][y][x][h][j]
 *
 * wattn_forward_gated -- wattn_forward_lse (lse may be NULL here) with that product fused into
 * the epilogue.
 *   gate_z : device pointer, [B][Hgrid][Wgrid][H][d] in q's element type (the gate logits, e.g.
 *            from wattn_cla_logits); read only; must not overlap out.  NULL: WATTN_ERR_NULL.
 *   lse    : the attention's row statistic (before the gate), as in wattn_forward_lse, or NULL.
 * dtype must be WATTN_BF16 or WATTN_BF16_OUT_FP32 (WATTN_ERR_DTYPE otherwise).  The sigmoid is
 * 1 / (1 + 2^(-z log2 e)) in fp32 with the hardware exp2 and reciprocal.  Other arguments,
 * checks and numerics are those of wattn_forward.
 */
int wattn_forward_gated(const void* q, const void* k, const void* v, void* out, float* lse, const void* gate_z,
                        int B, int H, int Hgrid, int Wgrid, int M, int shift, int d,
                        const float* theta, const void* bias_u, const void* bias_v, int r,
                        int dtype, void* stream);

/*
 * wattn_backward_gated -- wattn_backward for out = sigmoid(z) * attention (out as written by
 * wattn_forward_gated, lse from the same call), plus the gradient of the gate logits:
 *   the attention's output gradient is dout * sigmoid(z), rowsum(dout * out) equals the
 *   attention's rowsum(d_attention * attention), and
 *   dgate_z = dout * out * (1 - sigmoid(z))   (float32 [B][Hgrid][Wgrid][H][d], written).
 * gate_z, dgate_z : both required (WATTN_ERR_NULL); dgate_z must not overlap any other buffer.
 * All other arguments, checks and numerics are those of wattn_backward.
 */
int wattn_backward_gated(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, const void* gate_z, float* scratch, float* dq, float* dk, float* dv,
                         float* dtheta, float* dgate_z, int B, int H, int Hgrid, int Wgrid, int M, int shift,
                         int d, const float* theta, const void* bias_u, const void* bias_v, int r,
                         float* dbias_u, float* dbias_v, int dtype, void* stream);

/*
 * wattn_cla_logits -- the gate logits z = PW(DW3x3(x)) of the same section:
 *   y[b][i][j][c] = b_dw[c] + sum_{di,dj in -1..1} w_dw[c][di+1][dj+1] x[b][i+di][j+dj][c]
 *                   (x = 0 outside the grid: stride 1, zero padding 1, output the input's size)
 *   z[b][i][j][o] = b_pw[o] + sum_c w_pw[o][c] y[b][i][j][c]
 * with no activation between the two.
 *
 * x     : bfloat16 device pointer, [B][Hgrid][Wgrid][C] (channels last; with C = H * d this is
 *         the attention's [B][Hgrid][Wgrid][H][d] layout, channel c = h * d + j); read only.
 * w_dw  : float32 [C][3][3]; b_dw : float32 [C] or NULL (zero); w_pw : float32 [C][C] (output
 *         channel major); b_pw : float32 [C] or NULL.  Device pointers, read only.
 * z     : bfloat16 device pointer, [B][Hgrid][Wgrid][C], written; must not overlap an input.
 * C     : 32 .. 256, a multiple of 32 (WATTN_ERR_HEAD_DIM otherwise).  dtype : WATTN_BF16.
 * B * Hgrid * Wgrid must stay below 2^31 tokens (WATTN_ERR_SHAPE).
 * Numerics: the depth-wise sums in fp32, rounded to fp16 for the point-wise product (fp16
 * matrix cores, fp32 accumulation; w_pw rounded to fp16), z rounded once to bf16.  Depth-wise
 * outputs and w_pw entries must stay below 65504 in magnitude.
 */
int wattn_cla_logits(const void* x, const float* w_dw, const float* b_dw, const float* w_pw, const float* b_pw,
                     void* z, int B, int Hgrid, int Wgrid, int C, int dtype, void* stream);

/*
 * Gated local path of hybrid linear/softmax attention (HSMLA: Hierarchical Softmax
 * Multi-scale Linear Attention for Efficient Vision Transformers, technical summary section 2).
 * The global path is ReLU linear attention over all tokens; a learned gate shared by the heads
 * scores every spatial block, and only the blocks whose gate exceeds a threshold tau are routed
 * to a local softmax path inside a small w x w window, whose output becomes the global output
 * plus the residual R = O_local - O_lin-local.  Blocks are the w x w windows of the unshifted
 * grid, numbered blk = b * (Hgrid/w) * (Wgrid/w) + wy * (Wgrid/w) + wx.
 */

/*
 * wattn_select_blocks -- routing: list the blocks whose gate value exceeds tau.
 *
 * gate   : float32 device pointer, [nblocks] gate values (the gate network's M_b per block,
 *          in block order); read only.  A NaN gate is never selected; the comparison is
 *          strict (gate == tau is not selected).
 * nblocks: 1 .. WATTN_MAX_BLOCKS (WATTN_ERR_SHAPE otherwise).
 * list   : int32 device pointer, capacity nblocks; receives the selected block indices in
 *          ascending order in list[0 .. *count).  Entries past the count are left as they were.
 * count  : int32 device pointer to one element; receives the number selected.
 * None of gate, list and count may overlap (WATTN_ERR_ALIAS).  One workgroup launched on
 * `stream`; nothing is allocated.
 */
int wattn_select_blocks(const float* gate, int nblocks, float tau, int* list, int* count, void* stream);

/*
 * wattn_local_residual -- the residual correction of the listed blocks, in place:
 *
 *   out[t][h] += O_local[t][h] - O_lin-local[t][h]   for every token t of every listed block
 *
 * with, over the keys j of the token's w x w block (scale d^-1/2, no shift, no mask, no RoPE):
 *   O_local     = sum_j softmax_j(q_t . k_j / sqrt(d)) v_j
 *   O_lin-local = sum_j (relu(q_t) . relu(k_j)) v_j / (sum_j relu(q_t) . relu(k_j) + eps)
 * Tokens of unlisted blocks are not touched: `out` is expected to hold the global path's
 * output on entry.
 *
 * q, k, v : bfloat16 device pointers, [B][Hgrid][Wgrid][H][d]; read only.
 * out     : device pointer of the same shape, bfloat16 (dtype WATTN_BF16) or float32
 *           (WATTN_BF16_OUT_FP32); read and written.  Must not overlap q, k, v, list or count.
 * list, count : the block list and its length on the device (as written by
 *           wattn_select_blocks, capacity B * (Hgrid/w) * (Wgrid/w)).  The count is clamped to
 *           [0, number of blocks] and list entries outside the grid are skipped.  The entries
 *           must be distinct (wattn_select_blocks writes them ascending): each listed block is
 *           updated in place by its own workgroups with no atomics, so a block listed twice is
 *           updated by two racing sets of workgroups and its result is undefined.
 * w       : block side, one of 4, 8, 12, 16; Hgrid and Wgrid multiples of w.
 * d       : 32.   eps : finite, >= 0 (WATTN_ERR_VALUE otherwise).
 * One workgroup per (block, head) is launched for every block of the grid; those past the
 * device-side count return at once, so the call needs no host synchronisation.
 *
 * Numerics: scores from exact bf16 products accumulated in fp32; softmax in fp32 with the
 * exact row max; P (<= 1) and v rounded to fp16 for the value product (v entries must stay
 * below 65504 in magnitude); relu(k)^T v and the key sums accumulated in fp32 and applied
 * through a bf16 high + low split; the residual added in fp32 and rounded once to out's type.
 */
int wattn_local_residual(const void* q, const void* k, const void* v, void* out, const int* list,
                         const int* count, int B, int H, int Hgrid, int Wgrid, int w, int d, float eps,
                         int dtype, void* stream);

/*
 * wattn_gated_local -- routing and residual correction in one launch: the blocks whose gate
 * exceeds tau (strictly; a NaN gate never) get out += O_local - O_lin-local exactly as in
 * wattn_local_residual; no list is produced.  Every (block, head) has a workgroup that reads
 * its block's gate and leaves at once unless the block is selected.
 *
 * gate : float32 device pointer, [B * (Hgrid/w) * (Wgrid/w)] gate values in block order;
 *        read only; must not overlap out.
 * All other arguments, checks and numerics are those of wattn_local_residual.
 */
int wattn_gated_local(const void* q, const void* k, const void* v, void* out, const float* gate, float tau,
                      int B, int H, int Hgrid, int Wgrid, int w, int d, float eps, int dtype, void* stream);

/*
 * Model steps around the window attention (FLASHSWIN page, "How it works": Swin's hierarchy is
 * kept, with an overlapping stem -- a convolution with kernel 2p - 1, stride p, padding p - 1 --
 * in place of the patch embedding).  Activations are token-major bfloat16 [tokens][channels];
 * linear weights bfloat16 [out][in]; biases, norm gains and norm biases float32.  Every call
 * validates on the host first, launches on `stream` and allocates nothing.
 */
#define WATTN_ACT_NONE 0
#define WATTN_ACT_GELU 1 /* exact GELU: 0.5 x (1 + erf(x / sqrt 2)) */

/*
 * wattn_linear -- y = act(x W^T + bias) (+ residual), fp32 accumulation on bf16 matrix cores.
 *   x : [M][K] bf16; W : [N][K] bf16; bias : [N] float32 or NULL; residual : bf16 laid out like
 *   y, or NULL (it may be y itself: an in-place residual update).
 *   y : bf16 (dtype WATTN_BF16) or float32 (WATTN_BF16_OUT_FP32: no act, no residual).  Output
 *       column n of token m goes to (n / split) * M * split + m * split + n % split: split = N
 *       gives a plain [M][N] matrix, split = C with N = 3C gives q, k, v as three [M][C] tensors.
 *   K % 32 == 0, N % 4 == 0, split % 4 == 0, N % split == 0 (WATTN_ERR_SHAPE); act one of
 *   WATTN_ACT_* (WATTN_ERR_VALUE).  y must not overlap x, W or bias (WATTN_ERR_ALIAS).
 */
int wattn_linear(const void* x, const void* W, const float* bias, const void* residual, void* y, int M, int N,
                 int K, int split, int act, int dtype, void* stream);

/*
 * wattn_layernorm -- y[t] = (x[t] - mean) / sqrt(var + eps) * gamma + beta over the C channels
 * of each of T tokens (biased variance from fp32 sums).  x, y : [T][C] bf16 (no overlap);
 * gamma, beta : [C] float32.  C % 8 == 0; eps > 0 and finite (WATTN_ERR_VALUE).
 */
int wattn_layernorm(const void* x, const float* gamma, const float* beta, void* y, int64_t T, int C, float eps,
                    void* stream);

/*
 * wattn_patch_merge_norm -- the gather and norm of patch merging: output token (b, i, j) of
 * [B][Hgrid/2][Wgrid/2] is the layer norm of the 4C vector concatenating input tokens
 * (2i, 2j), (2i+1, 2j), (2i, 2j+1), (2i+1, 2j+1) of x [B][Hgrid][Wgrid][C].  y : [..][4C] bf16;
 * gamma, beta : [4C] float32.  Hgrid, Wgrid even; the 4C -> 2C reduction is a wattn_linear.
 */
int wattn_patch_merge_norm(const void* x, const float* gamma, const float* beta, void* y, int B, int Hgrid,
                           int Wgrid, int C, float eps, void* stream);

/*
 * wattn_stem_conv -- the overlapping stem: y[b][i][j][o] = bias[o] + sum_{c, di, dj < 2p-1}
 * W[o][c][di][dj] img[b][p i + di - (p-1)][p j + dj - (p-1)][c], zero outside the image.
 *   img : [B][Himg][Wimg][Cin] bf16 (NHWC); W : [Cout][Cin][2p-1][2p-1] bf16; bias : [Cout]
 *   float32; y : [B][Himg/p][Wimg/p][Cout] bf16.  Himg, Wimg multiples of p; Cout % 32 == 0; the
 *   weights must fit 64 KB as float32 ((2p-1)^2 Cin Cout <= 16384).  fp32 sums.
 */
int wattn_stem_conv(const void* img, const void* W, const float* bias, void* y, int B, int Himg, int Wimg, int Cin,
                    int Cout, int p, void* stream);

/* wattn_token_mean -- y[b][c] = mean over the n tokens of x[b][.][c]; x [B][n][C], y [B][C] bf16;
 * C % 8 == 0, B <= 65535 (fp32 sums, one rounding). */
int wattn_token_mean(const void* x, void* y, int B, int n, int C, void* stream);

/* Parameters of one pre-norm transformer block (device pointers; theta may be NULL). */
typedef struct {
  const float* ln1_g;  /* [C] */
  const float* ln1_b;  /* [C] */
  const void* w_qkv;   /* [3C][C] bf16: rows 0..C-1 give q, C..2C-1 k, 2C..3C-1 v (head h = c / 32) */
  const float* b_qkv;  /* [3C] or NULL */
  const void* w_proj;  /* [C][C] bf16 */
  const float* b_proj; /* [C] or NULL */
  const float* ln2_g;  /* [C] */
  const float* ln2_b;  /* [C] */
  const void* w_fc1;   /* [4C][C] bf16 */
  const float* b_fc1;  /* [4C] or NULL */
  const void* w_fc2;   /* [C][4C] bf16 */
  const float* b_fc2;  /* [C] or NULL */
  const float* theta;  /* [H][16] RoPE frequencies, or NULL */
} wattn_block_params_t;

/* Workspace bytes wattn_swin_block needs (10 * B * Hgrid * Wgrid * C); -1 for bad sizes. */
int64_t wattn_swin_block_workspace(int B, int Hgrid, int Wgrid, int C);

/*
 * wattn_swin_block -- one pre-norm block in place on x [B][Hgrid][Wgrid][C] bf16 (C = 32 H):
 *   x += proj(attention(LN1(x)))      attention: wattn_forward with window M, shift, theta
 *   x += fc2(GELU(fc1(LN2(x))))       (norm eps 1e-5, MLP width 4C)
 * workspace : device memory of at least wattn_swin_block_workspace(...) bytes (caller-owned,
 * scratch); it must not overlap x.  Seven kernels on `stream`.  Sizes follow wattn_forward.
 */
int wattn_swin_block(void* x, const wattn_block_params_t* p, void* workspace, int64_t workspace_bytes, int B,
                     int Hgrid, int Wgrid, int C, int H, int M, int shift, void* stream);

/*
 * wattn_pair_count -- number of (query, key) pairs with a finite logit in a call with
 * these sizes (the masked pairs of wrapped windows excluded).  Pure host arithmetic:
 * no HIP call, no side effect.  Returns -1 for sizes wattn_forward would reject with
 * WATTN_ERR_SHAPE or WATTN_ERR_SHIFT.
 */
int64_t wattn_pair_count(int B, int H, int Hgrid, int Wgrid, int M, int shift);

/* Human-readable name of a status code (static storage; never NULL). */
const char* wattn_status_string(int status);

/* WATTN_ABI_VERSION of the loaded library. */
int wattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WATTN_H */
