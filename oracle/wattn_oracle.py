"""Plain CPU oracle for shifted-window softmax attention with window-local 2D RoPE and an
explicit low-rank relative-position bias.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library and never imports its binding.

Everything is computed in float64 on the exact values of the (already dtype-rounded)
inputs.  The score matrix of every window is materialised, the bias is added as an
explicit N x N matrix U V^T, the shift mask is added as an explicit {0, -inf} matrix,
and a plain row softmax follows.  There is no tiling, no online softmax and no folding:
the fused operator is claimed to reach exactly this result (FlashSwin page,
"How it works", first change: the fused kernel is exact softmax attention, not an
approximation).

Sources (page title, section):
  [FS]  FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers
        with Memory Efficient Attention -- "What it is" (windowed attention materialises
        M^2 x M^2 scores per window) and "How it works" (second change: window-local
        2D RoPE, theta = exp(omega), first half of d encodes y and second half x, one
        shared frequency set, R(p)^T R(p') = R(p' - p); coordinates recomputed per window
        after the cyclic shift; wrapped windows masked additively).
  [RIB] Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution Transformer with
        FlashAttention -- technical summary, section 2.1 ([Q_c, Q_p][K_c, K_p]^T =
        Q_c K_c^T + Q_p K_p^T).

Readings where the pages leave a step open (each also used by the device library):
  * scale d^-1/2 on the content logits only; the bias U V^T is added unscaled;
  * window-local integer coordinates (row r, column c) in [0, M), not centred;
  * cyclic shift = Swin's roll by -s: rolled[Y] = original[(Y + s) mod Hg], output rolled back;
  * wrapped-window mask = per-axis region labels of the rolled coordinate
    (0: Y < G - M, 1: G - M <= Y < G - s, 2: Y >= G - s); a pair is masked (-inf)
    iff the labels differ on either axis;
  * RoPE rotates adjacent pairs (2j, 2j+1) by +phi for both q and k; pair j < d/4 uses
    phi = r * theta[j] (first half, y), pair j >= d/4 uses phi = c * theta[j] (second
    half, x); theta is passed as a per-pair table of d/2 entries per head.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------------------
# Geometry: windows, cyclic shift and region labels          [FS] "How it works"
# --------------------------------------------------------------------------------------

def local_coords(M: int):
    """Window-local (row, col) of token n = row*M + col, n in [0, M*M)."""
    n = np.arange(M * M)
    return n // M, n % M


def window_token_coords(Hg: int, Wg: int, M: int, shift: int, wy: int, wx: int):
    """Coordinates of the tokens of window (wy, wx) of the cyclically shifted grid.

    Returns (Y, X, y, x, r, c): rolled-grid coordinates, original-grid coordinates and
    window-local coordinates, each an int array of length M*M in local row-major order.
    The shift rolls the grid by -shift on both axes: the token shown at rolled position
    Y came from original row (Y + shift) mod Hg.
    """
    r, c = local_coords(M)
    Y = wy * M + r
    X = wx * M + c
    y = (Y + shift) % Hg
    x = (X + shift) % Wg
    return Y, X, y, x, r, c


def region_label(P: np.ndarray, G: int, M: int, shift: int) -> np.ndarray:
    """Region label of rolled coordinate P on an axis of length G (0, 1 or 2).

    With shift s > 0 the last band of windows (P >= G - M) holds two strips: tokens that
    were already there (label 1) and tokens that wrapped around from the start of the
    axis (P >= G - s, label 2).  Every other position has label 0.  With s = 0 all
    labels are 0.
    """
    P = np.asarray(P)
    if shift == 0:
        return np.zeros_like(P)
    return np.where(P < G - M, 0, np.where(P < G - shift, 1, 2))


def shift_mask(Y: np.ndarray, X: np.ndarray, Hg: int, Wg: int, M: int, shift: int) -> np.ndarray:
    """Explicit additive mask of one window: 0 where query and key share a region on both
    axes, -inf otherwise ([FS] "How it works": wrapped windows are masked additively)."""
    ly = region_label(Y, Hg, M, shift)
    lx = region_label(X, Wg, M, shift)
    same = (ly[:, None] == ly[None, :]) & (lx[:, None] == lx[None, :])
    return np.where(same, 0.0, NEG_INF)


# --------------------------------------------------------------------------------------
# Window-local 2D RoPE                                        [FS] "How it works", 2nd
# --------------------------------------------------------------------------------------

def rope_angles(theta_h: np.ndarray, r: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Rotation angle of every (token, pair): [len(r), d/2].

    Pair j < d/4 lies in the first half of the head dimension and encodes the vertical
    coordinate: angle r * theta[j].  Pair j >= d/4 lies in the second half and encodes
    the horizontal coordinate: angle c * theta[j].
    """
    th = np.asarray(theta_h, dtype=np.float64)
    d2 = th.shape[0]
    d4 = d2 // 2
    r = np.asarray(r, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    ang = np.empty((r.shape[0], d2), dtype=np.float64)
    ang[:, :d4] = r[:, None] * th[None, :d4]
    ang[:, d4:] = c[:, None] * th[None, d4:]
    return ang


def rope_rotate(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate each adjacent pair (x[2j], x[2j+1]) of every row by ang[:, j] (counter-
    clockwise): (a, b) -> (a cos - b sin, a sin + b cos)."""
    x = np.asarray(x, dtype=np.float64)
    a = x[..., 0::2]
    b = x[..., 1::2]
    cs = np.cos(ang)
    sn = np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = a * cs - b * sn
    out[..., 1::2] = a * sn + b * cs
    return out


# --------------------------------------------------------------------------------------
# One window, one head
# --------------------------------------------------------------------------------------

def window_logits(qw, kw, r, c, theta_h=None, u_h=None, v_h=None) -> np.ndarray:
    """Materialised N x N logits of one window and head (before the mask).

    S = (R q)(R k)^T / sqrt(d) + U V^T, with the rotation skipped when theta_h is None
    and the bias skipped when u_h is None.  The bias is an explicit matrix product of
    the two factors ([RIB] section 2.1 gives Q_c K_c^T + Q_p K_p^T).
    """
    qw = np.asarray(qw, dtype=np.float64)
    kw = np.asarray(kw, dtype=np.float64)
    d = qw.shape[-1]
    if theta_h is not None:
        ang = rope_angles(theta_h, r, c)
        qw = rope_rotate(qw, ang)
        kw = rope_rotate(kw, ang)
    S = (qw @ kw.T) / math.sqrt(d)
    if u_h is not None:
        u_h = np.asarray(u_h, dtype=np.float64)
        v_h = np.asarray(v_h, dtype=np.float64)
        S = S + u_h @ v_h.T
    return S


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax exp(S - max) / sum; -inf entries get weight exactly 0."""
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def window_weights(q, k, M, shift, b, wy, wx, h, theta=None, bias_u=None, bias_v=None):
    """Attention weights P (N x N) of window (wy, wx), head h, image b, plus the original
    coordinates (y, x) of its tokens in local order."""
    B, Hg, Wg, H, d = q.shape
    Y, X, y, x, r, c = window_token_coords(Hg, Wg, M, shift, wy, wx)
    qw = np.asarray(q[b, y, x, h, :], dtype=np.float64)
    kw = np.asarray(k[b, y, x, h, :], dtype=np.float64)
    th = None if theta is None else np.asarray(theta, dtype=np.float64)[h]
    uh = None if bias_u is None else np.asarray(bias_u, dtype=np.float64)[h]
    vh = None if bias_v is None else np.asarray(bias_v, dtype=np.float64)[h]
    S = window_logits(qw, kw, r, c, th, uh, vh)
    if shift > 0:
        S = S + shift_mask(Y, X, Hg, Wg, M, shift)
    return softmax_rows(S), y, x


def window_head_output(q, k, v, M, shift, b, wy, wx, h, theta=None, bias_u=None, bias_v=None):
    """Output rows (N x d, float64) of one window and head, with their original (y, x)."""
    P, y, x = window_weights(q, k, M, shift, b, wy, wx, h, theta, bias_u, bias_v)
    vw = np.asarray(v[b, y, x, h, :], dtype=np.float64)
    return P @ vw, y, x


def window_attention(q, k, v, M, shift=0, theta=None, bias_u=None, bias_v=None) -> np.ndarray:
    """Full shifted-window attention, float64 output of shape [B, Hg, Wg, H, d].

    q, k, v: [B, Hg, Wg, H, d]; theta: [H, d/2] or None; bias_u, bias_v: [H, M*M, r] or
    None.  Every window of every image and head is computed independently: gather the
    window's tokens, rotate, form the explicit logits, add the bias and mask matrices,
    softmax, multiply by V and write each row back to its token's original position
    (which also undoes the cyclic shift).
    """
    q = np.asarray(q)
    B, Hg, Wg, H, d = q.shape
    if Hg % M or Wg % M:
        raise ValueError("grid must be a multiple of the window size")
    if not 0 <= shift < M:
        raise ValueError("shift must lie in [0, M)")
    out = np.zeros((B, Hg, Wg, H, d), dtype=np.float64)
    th = _f64(theta)
    bu = _f64(bias_u)
    bv = _f64(bias_v)
    for b in range(B):
        for wy in range(Hg // M):
            for wx in range(Wg // M):
                for h in range(H):
                    o, y, x = window_head_output(q, k, v, M, shift, b, wy, wx, h, th, bu, bv)
                    out[b, y, x, h, :] = o
    return out


def unmasked_pairs(B, H, Hg, Wg, M, shift) -> int:
    """Number of (query, key) pairs with a finite logit over the whole job."""
    total = 0
    for wy in range(Hg // M):
        for wx in range(Wg // M):
            Y, X, _, _, _, _ = window_token_coords(Hg, Wg, M, shift, wy, wx)
            if shift > 0:
                total += int(np.isfinite(shift_mask(Y, X, Hg, Wg, M, shift)).sum())
            else:
                total += (M * M) ** 2
    return total * B * H


# --------------------------------------------------------------------------------------
# Row statistic and backward pass (gradients of a scalar loss sum(dout * out))
# --------------------------------------------------------------------------------------

def window_attention_lse(q, k, M, shift=0, theta=None, bias_u=None, bias_v=None) -> np.ndarray:
    """Natural-log log-sum-exp of every query row's logits (masked logits excluded):
    lse[b, y, x, h] = log sum_m exp(S[n, m]) for the query stored at original (y, x)."""
    q = np.asarray(q)
    B, Hg, Wg, H, d = q.shape
    out = np.zeros((B, Hg, Wg, H), dtype=np.float64)
    th, bu, bv = _f64(theta), _f64(bias_u), _f64(bias_v)
    for b in range(B):
        for wy in range(Hg // M):
            for wx in range(Wg // M):
                Y, X, y, x, r, c = window_token_coords(Hg, Wg, M, shift, wy, wx)
                for h in range(H):
                    S = window_logits(q[b, y, x, h, :], np.asarray(k)[b, y, x, h, :], r, c,
                                      None if th is None else th[h], None if bu is None else bu[h],
                                      None if bv is None else bv[h])
                    if shift > 0:
                        S = S + shift_mask(Y, X, Hg, Wg, M, shift)
                    m = np.max(S, axis=-1)
                    out[b, y, x, h] = m + np.log(np.sum(np.exp(S - m[:, None]), axis=-1))
    return out


def _rope_rotate_back(g: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Gradient through rope_rotate: the transpose of the rotation (rotate by -ang)."""
    return rope_rotate(g, -ang)


def _pair_cross(g: np.ndarray, xr: np.ndarray) -> np.ndarray:
    """d(loss)/d(angle) of every (row, pair) for a rotated vector xr with gradient g:
    the derivative of a rotation by phi is the rotation followed by a quarter turn,
    (a, b) -> (-b, a), so d/dphi = g . J xr = -g[2j] xr[2j+1] + g[2j+1] xr[2j]."""
    return -g[..., 0::2] * xr[..., 1::2] + g[..., 1::2] * xr[..., 0::2]


def window_attention_backward(q, k, v, dout, M, shift=0, theta=None, bias_u=None, bias_v=None):
    """Gradients of loss = sum(dout * window_attention(...)) with respect to every input.

    Returns a dict of float64 arrays: dq, dk, dv [B, Hg, Wg, H, d]; dtheta [H, d/2] (or
    None); dbias_u, dbias_v [H, M*M, r] (or None).  Per window and head it follows the
    forward steps backwards on the materialised matrices:
      O = P V, P = softmax(S):        dV = P^T dO,  dP = dO V^T,
                                      dS = P * (dP - rowsum(dO * O))   (0 where masked),
      S = s (R q)(R k)^T + U V_b^T:    d(Rq) = s dS (Rk),  d(Rk) = s dS^T (Rq),
                                      dU = dS V_b,  dV_b = dS^T U,
      Rq = rotate(q, angle):          dq = rotate(d(Rq), -angle),
                                      d angle[n, j] = d(Rq)[n] . J (Rq)[n] on pair j,
      angle[n, j] = pos[n, j] theta[j]: dtheta[j] += pos[n, j] * d angle[n, j]
    (and the same for k), with s = d^-1/2 and pos the window-local row (first half of
    the pairs) or column (second half).  The bias factors are shared by all windows and
    images, so their gradients sum over them.
    """
    q = np.asarray(q)
    B, Hg, Wg, H, d = q.shape
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout, dtype=np.float64)
    th, bu, bv = _f64(theta), _f64(bias_u), _f64(bias_v)
    sc = 1.0 / math.sqrt(d)
    dq = np.zeros((B, Hg, Wg, H, d))
    dk = np.zeros((B, Hg, Wg, H, d))
    dv = np.zeros((B, Hg, Wg, H, d))
    dth = None if th is None else np.zeros_like(th)
    dbu = None if bu is None else np.zeros_like(bu)
    dbv = None if bv is None else np.zeros_like(bv)
    d4 = d // 4
    for b in range(B):
        for wy in range(Hg // M):
            for wx in range(Wg // M):
                Y, X, y, x, r, c = window_token_coords(Hg, Wg, M, shift, wy, wx)
                for h in range(H):
                    qw = np.asarray(q[b, y, x, h, :], dtype=np.float64)
                    kw = np.asarray(k[b, y, x, h, :], dtype=np.float64)
                    vw = np.asarray(v[b, y, x, h, :], dtype=np.float64)
                    go = dout[b, y, x, h, :]
                    if th is not None:
                        ang = rope_angles(th[h], r, c)
                        qr, kr = rope_rotate(qw, ang), rope_rotate(kw, ang)
                    else:
                        qr, kr = qw, kw
                    S = sc * (qr @ kr.T)
                    if bu is not None:
                        S = S + bu[h] @ bv[h].T
                    if shift > 0:
                        S = S + shift_mask(Y, X, Hg, Wg, M, shift)
                    P = softmax_rows(S)
                    O = P @ vw
                    dP = go @ vw.T
                    dS = P * (dP - np.sum(go * O, axis=-1, keepdims=True))
                    dv[b, y, x, h, :] = P.T @ go
                    dqr = sc * (dS @ kr)
                    dkr = sc * (dS.T @ qr)
                    if th is not None:
                        dq[b, y, x, h, :] = _rope_rotate_back(dqr, ang)
                        dk[b, y, x, h, :] = _rope_rotate_back(dkr, ang)
                        dang = _pair_cross(dqr, qr) + _pair_cross(dkr, kr)  # [N, d/2]
                        pos = np.concatenate([np.repeat(r[:, None], d4, 1), np.repeat(c[:, None], d4, 1)], 1)
                        dth[h] += np.sum(pos * dang, axis=0)
                    else:
                        dq[b, y, x, h, :] = dqr
                        dk[b, y, x, h, :] = dkr
                    if bu is not None:
                        dbu[h] += dS @ bv[h]
                        dbv[h] += dS.T @ bu[h]
    return {"dq": dq, "dk": dk, "dv": dv, "dtheta": dth, "dbias_u": dbu, "dbias_v": dbv}
