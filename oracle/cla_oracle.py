"""Plain CPU oracle for the convolutional gate on the attention output, and the cyclic
window schedule of a stack of window-attention layers.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library and never imports its binding.

Source (page title, section):
  [RIB] Rank-Factorized Implicit Neural Bias: Scaling Super-Resolution Transformer with
        FlashAttention -- section 2.2 (convolutional local attention: a 3x3 depth-wise and a
        1x1 point-wise convolution extract local features, a sigmoid turns them into a gating
        map, and the map modulates the attention output) and section 2.3 (cyclic window
        strategy: the window size changes from layer to layer, e.g. 16, 32, 64, 16, 32, 64).

Everything is float64 on the exact values of the (already dtype-rounded) inputs.

Readings where the page leaves a step open (each also used by the device library):
  * the convolutions read the layer's input feature map x ([B][Hg][Wg][C], C = H * d, channel
    c = h * d + j), not the attention output, so the gate does not depend on the attention;
  * the depth-wise convolution has a 3 x 3 kernel per channel, stride 1, zero padding 1 (the
    output has the input's size) and a bias per channel; the point-wise convolution is a
    C x C matrix plus a bias; there is no activation between them;
  * the gate acts on the attention output as an elementwise product: out = sigmoid(z) *
    attention output, channel by channel, with z the point-wise output (the gate logits);
  * a cyclic schedule runs the layers in order, layer l with window side M_l and shift 0 or
    M_l / 2 (alternating, as Swin does); each layer has its own q, k, v and parameters.
"""

from __future__ import annotations

import numpy as np

from .wattn_oracle import window_attention, window_attention_backward


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(z):
    """1 / (1 + e^-z), evaluated through e^-|z| so that no intermediate overflows."""
    z = _f64(z)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def depthwise3x3(x, w_dw, b_dw) -> np.ndarray:
    """y[b, i, j, c] = b_dw[c] + sum_{di, dj in -1..1} w_dw[c, di+1, dj+1] x[b, i+di, j+dj, c],
    with x = 0 outside the grid.  x: [B][Hg][Wg][C]; w_dw: [C][3][3]; b_dw: [C]."""
    x = _f64(x)
    B, Hg, Wg, C = x.shape
    xp = np.zeros((B, Hg + 2, Wg + 2, C))
    xp[:, 1:-1, 1:-1] = x
    y = np.broadcast_to(_f64(b_dw), x.shape).copy()
    w = _f64(w_dw)
    for di in range(3):
        for dj in range(3):
            y += w[:, di, dj] * xp[:, di:di + Hg, dj:dj + Wg]
    return y


def pointwise(y, w_pw, b_pw) -> np.ndarray:
    """z[..., o] = b_pw[o] + sum_c w_pw[o, c] y[..., c]."""
    return _f64(y) @ _f64(w_pw).T + _f64(b_pw)


def cla_gate_logits(x, w_dw, b_dw, w_pw, b_pw) -> np.ndarray:
    """The gate logits z = PW(DW3x3(x)) as [B][Hg][Wg][C]."""
    return pointwise(depthwise3x3(x, w_dw, b_dw), w_pw, b_pw)


def gated_window_attention(q, k, v, z, M, shift=0, theta=None, bias_u=None, bias_v=None) -> np.ndarray:
    """sigmoid(z) * window attention; z: [B][Hg][Wg][H][d] (channel c = h * d + j)."""
    return sigmoid(z) * window_attention(q, k, v, M, shift, theta, bias_u, bias_v)


def gated_window_attention_backward(q, k, v, z, dout, M, shift=0, theta=None, bias_u=None, bias_v=None):
    """Gradients of sum(dout * gated_window_attention(...)): the attention's gradients for the
    output gradient dout * sigmoid(z), plus dz = dout * attention * sigmoid'(z)."""
    s = sigmoid(z)
    attn = window_attention(q, k, v, M, shift, theta, bias_u, bias_v)
    g = window_attention_backward(q, k, v, _f64(dout) * s, M, shift, theta, bias_u, bias_v)
    g["dz"] = _f64(dout) * attn * s * (1.0 - s)
    return g


def cyclic_schedule(n_layers: int, sides=(16, 32, 64)):
    """(M, shift) per layer: the window sides in turn, shift 0 on even layers and M / 2 on odd."""
    out = []
    for l in range(n_layers):
        M = sides[l % len(sides)]
        out.append((M, 0 if l % 2 == 0 else M // 2))
    return out
