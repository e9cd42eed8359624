"""Plain CPU oracle for the model steps around the window attention: the overlapping stem,
layer norm, the linear layers of a transformer block, patch merging, and a whole FlashSwin-T
forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP library and never imports its binding.

Source (page title, section):
  [FS]  FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with
        Memory Efficient Attention -- "How it works": the hierarchy and attention pattern of
        Swin are kept and three parts change: the fused window attention, window-local 2D
        RoPE in place of the relative-position bias, and an overlapping stem (a convolution
        with kernel 2p - 1, stride p and padding p - 1 in place of the non-overlapping patch
        embedding).  "What is different": throughput of FlashSwin-T in img/s at patch 4 and 2.

Everything is float64 on the exact values of the inputs; every intermediate is kept in float64.

Readings where the pages leave a step open (the pages keep Swin's hierarchy without spelling
it out; each reading is also used by the device library):
  * the block is the pre-norm Swin block: x += proj(attn(LN1(x))), x += fc2(GELU(fc1(LN2(x))));
    attention is the window attention of the other oracle (scale d^-1/2, window-local RoPE,
    cyclic shift on every second block), the MLP widens by 4, GELU is the exact erf form,
    layer norm has eps = 1e-5 and an affine gain and bias, every linear layer has a bias except
    the patch-merging reduction;
  * qkv projection: one C -> 3C linear layer whose outputs are q, k, v in that order, each
    split into heads h = 0 .. H-1 of d channels (channel c of q is head c // d, dim c % d);
  * the stem is the convolution above on an NHWC image with 3 channels, followed by a layer
    norm over the embedding (Swin's patch norm);
  * patch merging concatenates the 2 x 2 neighbours (y, x), (y+1, x), (y, x+1), (y+1, x+1) in
    that order, normalises the 4C vector and maps it to 2C without bias;
  * FlashSwin-T: C = 96, depths 2, 2, 6, 2, heads 3, 6, 12, 24 (d = 32), a final layer norm,
    global average pooling and a linear head; a stage whose grid side is not above the window
    side M uses one window over the grid and no shift.
"""

from __future__ import annotations

import math

import numpy as np

from .wattn_oracle import window_attention


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def layernorm(x, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * gamma + beta over the last axis (biased variance)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def linear(x, W, b=None) -> np.ndarray:
    """x W^T + b; W is [out][in]."""
    y = _f64(x) @ _f64(W).T
    return y if b is None else y + _f64(b)


def gelu(x) -> np.ndarray:
    from scipy.special import erf

    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def stem_conv(img, W, b, p: int) -> np.ndarray:
    """Overlapping patch embedding: kernel k = 2p - 1, stride p, zero padding p - 1.
    img: [B][Himg][Wimg][Cin]; W: [Cout][Cin][k][k]; b: [Cout].  Returns [B][Himg/p][Wimg/p][Cout]."""
    img = _f64(img)
    B, Hi, Wi, Cin = img.shape
    k = 2 * p - 1
    pad = p - 1
    Ho, Wo = (Hi + 2 * pad - k) // p + 1, (Wi + 2 * pad - k) // p + 1
    xp = np.zeros((B, Hi + 2 * pad, Wi + 2 * pad, Cin))
    xp[:, pad:pad + Hi, pad:pad + Wi] = img
    W = _f64(W)
    out = np.broadcast_to(_f64(b), (B, Ho, Wo, W.shape[0])).copy()
    for di in range(k):
        for dj in range(k):
            patch = xp[:, di:di + p * (Ho - 1) + 1:p, dj:dj + p * (Wo - 1) + 1:p]   # [B][Ho][Wo][Cin]
            out += patch @ W[:, :, di, dj].T
    return out


def patch_merge(x, gamma, beta, W) -> np.ndarray:
    """[B][Hg][Wg][C] -> [B][Hg/2][Wg/2][2C]: 2 x 2 neighbours concatenated, normalised, reduced."""
    x = _f64(x)
    cat = np.concatenate([x[:, 0::2, 0::2], x[:, 1::2, 0::2], x[:, 0::2, 1::2], x[:, 1::2, 1::2]], axis=-1)
    return linear(layernorm(cat, gamma, beta), W)


def swin_block(x, P: dict, H: int, M: int, shift: int, theta=None) -> np.ndarray:
    """One pre-norm block on [B][Hg][Wg][C]; P holds ln1_g, ln1_b, w_qkv, b_qkv, w_proj, b_proj,
    ln2_g, ln2_b, w_fc1, b_fc1, w_fc2, b_fc2."""
    x = _f64(x)
    B, Hg, Wg, C = x.shape
    d = C // H
    qkv = linear(layernorm(x, P["ln1_g"], P["ln1_b"]), P["w_qkv"], P["b_qkv"])
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, Hg, Wg, H, d) for i in range(3))
    a = window_attention(q, k, v, M, shift, theta).reshape(B, Hg, Wg, C)
    x = x + linear(a, P["w_proj"], P["b_proj"])
    h = gelu(linear(layernorm(x, P["ln2_g"], P["ln2_b"]), P["w_fc1"], P["b_fc1"]))
    return x + linear(h, P["w_fc2"], P["b_fc2"])


def stage_window(grid: int, M: int, shift: int):
    """(window side, shift) of a stage: one window over the grid and no shift when the grid side
    is not above M."""
    return (grid, 0) if grid <= M else (M, shift)


def flashswin_forward(img, params: dict, p: int, M: int) -> np.ndarray:
    """Class logits [B][n_classes] of the FlashSwin-T forward pass (see the module readings).
    params: stem_w, stem_b, stem_ln_g, stem_ln_b; stages[s] = dict(blocks=[block dicts],
    theta=[H][d/2], merge=None or dict(ln_g, ln_b, w)); norm_g, norm_b, head_w, head_b."""
    x = stem_conv(img, params["stem_w"], params["stem_b"], p)
    x = layernorm(x, params["stem_ln_g"], params["stem_ln_b"])
    for st in params["stages"]:
        B, Hg, Wg, C = x.shape
        H = st["heads"]
        for i, blk in enumerate(st["blocks"]):
            Mw, s = stage_window(Hg, M, 0 if i % 2 == 0 else M // 2)
            x = swin_block(x, blk, H, Mw, s, st["theta"])
        if st.get("merge") is not None:
            m = st["merge"]
            x = patch_merge(x, m["ln_g"], m["ln_b"], m["w"])
    x = layernorm(x, params["norm_g"], params["norm_b"])
    return linear(x.mean(axis=(1, 2)), params["head_w"], params["head_b"])
