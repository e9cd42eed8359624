"""Pins of the oracle's backward pass and row statistic (CPU only).

The oracle's gradients are checked against things that do not use its backward formulas:
central finite differences of the oracle's own forward pass, torch autograd (float64, CPU)
through an independent formulation of the shifted layer (roll, reshape into windows,
region-label mask, explicit RoPE, bias matrix, softmax), and closed forms.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from inputs import theta_table
from torch_layer import torch_layer as _torch_layer


def _rng(seed):
    return np.random.default_rng(seed)


def _loss(q, k, v, dout, M, s, th, U, V):
    return float(np.sum(dout * oracle.window_attention(q, k, v, M, s, th, U, V)))


def test_backward_matches_central_differences():
    rng = _rng(101)
    B, Hg, Wg, M, s, H, d, r = 1, 8, 8, 4, 2, 1, 8, 2
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    th = theta_table(H, d, 0.3, 102).astype(np.float64) * 3.0  # large angles: every pair rotates visibly
    U = rng.normal(size=(H, M * M, r))
    V = rng.normal(size=(H, M * M, r))
    dout = rng.normal(size=(B, Hg, Wg, H, d))
    g = oracle.window_attention_backward(q, k, v, dout, M, s, th, U, V)
    args = {"q": q, "k": k, "v": v, "theta": th, "bias_u": U, "bias_v": V}
    names = {"q": "dq", "k": "dk", "v": "dv", "theta": "dtheta", "bias_u": "dbias_u", "bias_v": "dbias_v"}
    eps = 1e-6
    for name, arr in args.items():
        flat = arr.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 20), replace=False)
        for i in idx:
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(args["q"], args["k"], args["v"], dout, M, s, args["theta"], args["bias_u"], args["bias_v"])
            flat[i] = keep - eps
            lm = _loss(args["q"], args["k"], args["v"], dout, M, s, args["theta"], args["bias_u"], args["bias_v"])
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            an = g[names[name]].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (name, i, fd, an)


@pytest.mark.parametrize("Hg,Wg,M,s", [(8, 8, 4, 2), (8, 12, 4, 1), (12, 8, 4, 3), (8, 8, 8, 0), (16, 8, 8, 5)])
def test_backward_matches_torch_autograd(Hg, Wg, M, s):
    rng = _rng(200 + Hg + Wg + M + s)
    B, H, d, r = 2, 2, 8, 2
    q, k, v, dout = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(4))
    th = theta_table(H, d, 0.2, 7).astype(np.float64) * 2.0
    th[1] *= 0.5  # heads with different tables
    U, V = rng.normal(size=(H, M * M, r)), rng.normal(size=(H, M * M, r))
    g = oracle.window_attention_backward(q, k, v, dout, M, s, th, U, V)
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v, th, U, V)]
    out, lse = _torch_layer(*ts, M, s)
    (out * torch.from_numpy(dout)).sum().backward()
    for t, name in zip(ts, ("dq", "dk", "dv", "dtheta", "dbias_u", "dbias_v")):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
    np.testing.assert_allclose(oracle.window_attention_lse(q, k, M, s, th, U, V), lse.detach().numpy(),
                               rtol=1e-12, atol=1e-12)


def test_value_gradient_sums_to_output_gradient_per_window():
    """Every query's weights sum to one over the keys of its window, so the value
    gradients of a window sum to the output gradients of the same window."""
    rng = _rng(301)
    B, Hg, Wg, M, s, H, d = 2, 8, 12, 4, 3, 2, 8
    q, k, v, dout = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(4))
    th = theta_table(H, d, 0.1, 3)
    g = oracle.window_attention_backward(q, k, v, dout, M, s, th)
    for wy in range(Hg // M):
        for wx in range(Wg // M):
            _, _, y, x, _, _ = oracle.window_token_coords(Hg, Wg, M, s, wy, wx)
            np.testing.assert_allclose(g["dv"][:, y, x].sum(axis=1), dout[:, y, x].sum(axis=1), atol=1e-12)


def test_zero_output_gradient_gives_zero_gradients():
    rng = _rng(302)
    B, Hg, Wg, M, s, H, d, r = 1, 8, 8, 4, 2, 2, 8, 2
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    U, V = rng.normal(size=(H, M * M, r)), rng.normal(size=(H, M * M, r))
    g = oracle.window_attention_backward(q, k, v, np.zeros_like(q), M, s, theta_table(H, d, 0.1, 4), U, V)
    for name, a in g.items():
        assert np.all(a == 0.0), name


def test_lse_of_equal_logits_is_log_region_size():
    """With q = 0 and no bias every logit of a row is 0, so the row statistic is the log of
    the number of keys the query sees: its region of the shifted window."""
    B, Hg, Wg, M, s, H, d = 1, 8, 8, 4, 1, 1, 8
    q = np.zeros((B, Hg, Wg, H, d))
    k = _rng(303).normal(size=(B, Hg, Wg, H, d))
    lse = oracle.window_attention_lse(q, k, M, s, theta_table(H, d, 0.1, 5))
    for y in range(Hg):
        for x in range(Wg):
            # rolled coordinate of original (y, x) and its region along each axis
            Y, X = (y - s) % Hg, (x - s) % Wg
            ny = M if Y < Hg - M else (M - s if Y < Hg - s else s)
            nx = M if X < Wg - M else (M - s if X < Wg - s else s)
            assert abs(lse[0, y, x, 0] - math.log(ny * nx)) < 1e-12
