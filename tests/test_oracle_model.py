"""Pins of the model-step oracle (CPU only): layer norm, linear layers, GELU and the stem
against torch's functional ops, patch merging against a reshape formulation, the block and the
whole forward pass against a torch re-implementation built on the independent window-attention
formulation of tests/torch_layer.py."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from inputs import ModelConfig, block_params, images, model_params, theta_table
from torch_layer import torch_layer


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def test_layernorm_linear_gelu_match_torch():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(5, 7, 48))
    g, b = rng.normal(size=48), rng.normal(size=48)
    np.testing.assert_allclose(oracle.layernorm(x, g, b), F.layer_norm(_t(x), (48,), _t(g), _t(b), 1e-5).numpy(),
                               rtol=1e-12, atol=1e-12)
    W, c = rng.normal(size=(20, 48)), rng.normal(size=20)
    np.testing.assert_allclose(oracle.linear(x, W, c), F.linear(_t(x), _t(W), _t(c)).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.gelu(x), F.gelu(_t(x)).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p,side", [(2, 8), (4, 16), (2, 6)])
def test_stem_matches_torch_conv2d(p, side):
    rng = np.random.default_rng(2 + p)
    k = 2 * p - 1
    img = rng.normal(size=(2, side, side, 3))
    W, b = rng.normal(size=(8, 3, k, k)), rng.normal(size=8)
    ref = F.conv2d(_t(img).permute(0, 3, 1, 2), _t(W), _t(b), stride=p, padding=p - 1).permute(0, 2, 3, 1).numpy()
    got = oracle.stem_conv(img, W, b, p)
    assert got.shape == (2, side // p, side // p, 8)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_patch_merge_matches_reshape_formulation():
    rng = np.random.default_rng(3)
    B, Hg, Wg, C = 2, 6, 8, 4
    x = rng.normal(size=(B, Hg, Wg, C))
    g, b, W = rng.normal(size=4 * C), rng.normal(size=4 * C), rng.normal(size=(2 * C, 4 * C))
    # [B, Hg/2, dy, Wg/2, dx, C] -> order (dx, dy): (0,0), (1,0), (0,1), (1,1) in (dy, dx) terms
    r = x.reshape(B, Hg // 2, 2, Wg // 2, 2, C).transpose(0, 1, 3, 4, 2, 5).reshape(B, Hg // 2, Wg // 2, 4 * C)
    ref = F.linear(F.layer_norm(_t(r), (4 * C,), _t(g), _t(b), 1e-5), _t(W)).numpy()
    np.testing.assert_allclose(oracle.patch_merge(x, g, b, W), ref, rtol=1e-12, atol=1e-12)


def _torch_block(x, P, H, M, s, theta):
    B, Hg, Wg, C = x.shape
    d = C // H
    T = lambda k: _t(P[k])
    h = F.layer_norm(x, (C,), T("ln1_g"), T("ln1_b"), 1e-5)
    qkv = F.linear(h, T("w_qkv"), T("b_qkv"))
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, Hg, Wg, H, d) for i in range(3))
    zero = torch.zeros((H, M * M, 1), dtype=torch.float64)
    a, _ = torch_layer(q, k, v, _t(theta), zero, zero, M, s)
    x = x + F.linear(a.reshape(B, Hg, Wg, C), T("w_proj"), T("b_proj"))
    h = F.gelu(F.linear(F.layer_norm(x, (C,), T("ln2_g"), T("ln2_b"), 1e-5), T("w_fc1"), T("b_fc1")))
    return x + F.linear(h, T("w_fc2"), T("b_fc2"))


@pytest.mark.parametrize("M,s", [(4, 0), (4, 2)])
def test_block_matches_torch_formulation(M, s):
    rng = np.random.default_rng(4 + s)
    B, Hg, Wg, C, H = 2, 8, 12, 16, 2
    x = rng.normal(size=(B, Hg, Wg, C))
    P = block_params(C, 5, "fp32")
    th = theta_table(H, C // H, 0.1, 6).astype(np.float64) * 3.0
    ref = _torch_block(_t(x), P, H, M, s, th).numpy()
    np.testing.assert_allclose(oracle.swin_block(x, P, H, M, s, th), ref, rtol=1e-10, atol=1e-10)


def test_stage_window_rule():
    assert oracle.stage_window(64, 32, 16) == (32, 16)
    assert oracle.stage_window(32, 32, 16) == (32, 0)
    assert oracle.stage_window(16, 32, 0) == (16, 0)


def test_forward_pass_matches_torch_formulation():
    """A miniature of the model (64 px, patch 4, two stages of widths 16 and 32, window 8): the
    oracle's forward pass against the same pass written with torch ops."""
    cfg = ModelConfig("mini", 2, 64, 4, 8, C=16, depths=(2, 2), heads=(2, 2), n_classes=10, seed=7)
    P = model_params(cfg, "fp32")
    img = images(2, 64, 8, "fp32").astype(np.float64)
    got = oracle.flashswin_forward(img, P, cfg.p, cfg.M)

    x = F.conv2d(_t(img).permute(0, 3, 1, 2), _t(P["stem_w"]), _t(P["stem_b"]), stride=4, padding=3)
    x = x.permute(0, 2, 3, 1)
    x = F.layer_norm(x, (16,), _t(P["stem_ln_g"]), _t(P["stem_ln_b"]), 1e-5)
    for st in P["stages"]:
        Hg = x.shape[1]
        for i, blk in enumerate(st["blocks"]):
            Mw, s = (Hg, 0) if Hg <= cfg.M else (cfg.M, 0 if i % 2 == 0 else cfg.M // 2)
            x = _torch_block(x, blk, st["heads"], Mw, s, st["theta"].astype(np.float64))
        if st["merge"] is not None:
            B, Hg, Wg, C = x.shape
            r = x.reshape(B, Hg // 2, 2, Wg // 2, 2, C).permute(0, 1, 3, 4, 2, 5).reshape(B, Hg // 2, Wg // 2, 4 * C)
            m = st["merge"]
            x = F.linear(F.layer_norm(r, (4 * C,), _t(m["ln_g"]), _t(m["ln_b"]), 1e-5), _t(m["w"]))
    x = F.layer_norm(x, (x.shape[-1],), _t(P["norm_g"]), _t(P["norm_b"]), 1e-5)
    ref = F.linear(x.mean(dim=(1, 2)), _t(P["head_w"]), _t(P["head_b"])).numpy()
    assert got.shape == (2, 10)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)
    assert math.isfinite(float(np.abs(got).sum()))
