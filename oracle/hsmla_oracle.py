"""Plain CPU oracle for the block-gated local softmax path of hybrid linear/softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library and never imports its binding.

Source (page title, section):
  [HS]  HSMLA: Hierarchical Softmax Multi-scale Linear Attention for Efficient Vision
        Transformers -- technical summary, section 2 (method): the global backbone is ReLU
        linear attention; a learned gate shared by all heads scores every spatial block and
        only blocks whose gate exceeds a threshold tau take the local softmax path; there,
        softmax attention runs inside a small w x w window and the output becomes the global
        linear output plus the residual R = O_local - O_lin-local.

Everything is float64 on the exact values of the (already dtype-rounded) inputs; scores and
linear-attention weights are materialised per window, nothing is tiled or reassociated.

Readings where the page leaves a step open (each also used by the device library):
  * a block is one w x w window of the unshifted window grid (the page's "contiguous
    spatial tile"); blocks are numbered b * nWy * nWx + wy * nWx + wx;
  * a block is selected iff its gate value is strictly greater than tau; the selected
    blocks form an ascending list (a NaN gate is never selected);
  * the feature map of the linear path is phi(x) = max(x, 0) per channel, and a query's
    linear output is sum_j (phi(q).phi(k_j)) v_j / (sum_j phi(q).phi(k_j) + eps), with eps
    a caller-supplied guard in the denominator;
  * O_lin-local is that linear attention with the keys restricted to the query's window,
    O_local the softmax attention over the same keys with scale d^-1/2, no shift, no mask,
    no RoPE and no bias;
  * the residual is added unscaled (hard routing): out = base + O_local - O_lin-local on the
    selected windows, out = base elsewhere, where base is the global path's output.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------------------
# Routing                                      [HS] section 2, hierarchical block-level gating
# --------------------------------------------------------------------------------------

def select_blocks(gate, tau: float) -> np.ndarray:
    """Ascending flat indices of the blocks whose gate value exceeds tau (strictly).

    gate: [B][nWy][nWx] gate values M_b in [0, 1] (any float dtype; compared as stored)."""
    g = np.asarray(gate).reshape(-1)
    return np.array([i for i in range(g.size) if g[i] > tau], dtype=np.int64)


def block_origin(block: int, nWy: int, nWx: int, w: int):
    """(b, y0, x0): image and top-left token of block `block` of the w x w window grid."""
    b, r = divmod(int(block), nWy * nWx)
    wy, wx = divmod(r, nWx)
    return b, wy * w, wx * w


# --------------------------------------------------------------------------------------
# The two attentions of one window                  [HS] section 2, two-path residual kernel
# --------------------------------------------------------------------------------------

def relu_linear_attention(qh, kh, vh, eps: float) -> np.ndarray:
    """ReLU linear attention of queries qh [n][d] over keys kh [m][d], values vh [m][d],
    written as the materialised weight matrix A[i][j] = phi(q_i) . phi(k_j)."""
    A = np.maximum(_f64(qh), 0.0) @ np.maximum(_f64(kh), 0.0).T
    return (A @ _f64(vh)) / (A.sum(axis=1, keepdims=True) + eps)


def softmax_attention(qh, kh, vh) -> np.ndarray:
    """Exact softmax attention with scale d^-1/2 (scores materialised)."""
    S = (_f64(qh) @ _f64(kh).T) / math.sqrt(qh.shape[-1])
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return (P / P.sum(axis=1, keepdims=True)) @ _f64(vh)


def window_tokens(q, block: int, w: int):
    """Index arrays (b, ys, xs) of the w*w tokens of a block, token n = i * w + j."""
    _, Hg, Wg, _, _ = q.shape
    b, y0, x0 = block_origin(block, Hg // w, Wg // w, w)
    n = np.arange(w * w)
    return b, y0 + n // w, x0 + n % w


def local_residual_window(q, k, v, block: int, w: int, eps: float) -> np.ndarray:
    """R = O_local - O_lin-local of every token and head of one block: [w*w][H][d]."""
    b, ys, xs = window_tokens(q, block, w)
    H = q.shape[3]
    R = np.empty((w * w, H, q.shape[4]))
    for h in range(H):
        qh, kh, vh = q[b, ys, xs, h], k[b, ys, xs, h], v[b, ys, xs, h]
        R[:, h] = softmax_attention(qh, kh, vh) - relu_linear_attention(qh, kh, vh, eps)
    return R


def local_residual(q, k, v, base, blocks, w: int, eps: float) -> np.ndarray:
    """out = base + R on the tokens of the listed blocks, base elsewhere ([B][Hg][Wg][H][d])."""
    B, Hg, Wg, H, d = q.shape
    if Hg % w or Wg % w:
        raise ValueError("grid not divisible by the window size")
    out = _f64(base).copy()
    for blk in blocks:
        b, ys, xs = window_tokens(q, int(blk), w)
        out[b, ys, xs] += local_residual_window(q, k, v, int(blk), w, eps)
    return out


def gated_local_path(q, k, v, base, gate, tau: float, w: int, eps: float) -> np.ndarray:
    """Routing followed by the residual correction of the selected blocks."""
    return local_residual(q, k, v, base, select_blocks(gate, tau), w, eps)


def global_linear_attention(q, k, v, eps: float) -> np.ndarray:
    """The global path: ReLU linear attention of every token over all tokens of its image
    and head ([HS] section 2, global backbone), weights materialised."""
    B, Hg, Wg, H, d = q.shape
    out = np.empty((B, Hg, Wg, H, d))
    for b in range(B):
        for h in range(H):
            qh = q[b, :, :, h].reshape(-1, d)
            kh = k[b, :, :, h].reshape(-1, d)
            vh = v[b, :, :, h].reshape(-1, d)
            out[b, :, :, h] = relu_linear_attention(qh, kh, vh, eps).reshape(Hg, Wg, d)
    return out
