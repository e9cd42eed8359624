"""Pins of the convolutional-gate oracle (CPU only): the convolutions against torch's conv2d,
the sigmoid's identities, the gated attention's limits, and its backward pass against torch
autograd through an independent formulation of the layer and against finite differences."""

import numpy as np
import pytest
import torch

import oracle
from inputs import theta_table
from torch_layer import torch_layer


def _rng(seed):
    return np.random.default_rng(seed)


def test_depthwise_matches_torch_conv2d():
    rng = _rng(1)
    B, Hg, Wg, C = 2, 7, 9, 6
    x = rng.normal(size=(B, Hg, Wg, C))
    w, b = rng.normal(size=(C, 3, 3)), rng.normal(size=C)
    ref = torch.nn.functional.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None],
                                     torch.from_numpy(b), padding=1, groups=C).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(oracle.depthwise3x3(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_pointwise_matches_torch_conv2d():
    rng = _rng(2)
    B, Hg, Wg, C = 2, 5, 4, 6
    y = rng.normal(size=(B, Hg, Wg, C))
    w, b = rng.normal(size=(C, C)), rng.normal(size=C)
    ref = torch.nn.functional.conv2d(torch.from_numpy(y).permute(0, 3, 1, 2), torch.from_numpy(w)[:, :, None, None],
                                     torch.from_numpy(b)).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(oracle.pointwise(y, w, b), ref, rtol=1e-12, atol=1e-12)


def test_gate_logits_of_a_single_impulse():
    """One nonzero input pixel: the depth-wise output is its kernel, flipped into place, and the
    point-wise output mixes those nine pixels' channels."""
    C = 3
    x = np.zeros((1, 5, 5, C))
    x[0, 2, 2] = [1.0, 2.0, -1.0]
    w = np.arange(C * 9, dtype=np.float64).reshape(C, 3, 3)
    y = oracle.depthwise3x3(x, w, np.zeros(C))
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            # output pixel (2 - di, 2 - dj) sees the impulse through tap (di + 1, dj + 1)
            np.testing.assert_allclose(y[0, 2 - di, 2 - dj], w[:, di + 1, dj + 1] * x[0, 2, 2])
    assert np.count_nonzero(np.abs(y).sum(axis=-1)) == 9


def test_sigmoid_identities():
    z = np.linspace(-30, 30, 121)
    s = oracle.sigmoid(z)
    np.testing.assert_allclose(s + oracle.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    assert oracle.sigmoid(0.0) == 0.5
    assert np.all(np.diff(s) > 0)


def test_gated_attention_limits():
    rng = _rng(3)
    B, Hg, Wg, H, d, M, s = 1, 8, 8, 2, 8, 4, 2
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    th = theta_table(H, d, 0.1, 4)
    att = oracle.window_attention(q, k, v, M, s, th)
    np.testing.assert_allclose(oracle.gated_window_attention(q, k, v, np.full(q.shape, 50.0), M, s, th), att,
                               rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(oracle.gated_window_attention(q, k, v, np.zeros(q.shape), M, s, th), 0.5 * att,
                               rtol=1e-15)
    assert np.all(np.abs(oracle.gated_window_attention(q, k, v, np.full(q.shape, -800.0), M, s, th)) == 0.0)


@pytest.mark.parametrize("Hg,Wg,M,s", [(8, 8, 4, 2), (8, 12, 4, 1)])
def test_gated_backward_matches_torch_autograd(Hg, Wg, M, s):
    rng = _rng(10 + Wg + s)
    B, H, d, r = 2, 2, 8, 2
    q, k, v, z, dout = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(5))
    th = theta_table(H, d, 0.2, 7).astype(np.float64) * 2.0
    U, V = rng.normal(size=(H, M * M, r)), rng.normal(size=(H, M * M, r))
    g = oracle.gated_window_attention_backward(q, k, v, z, dout, M, s, th, U, V)
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v, th, U, V, z)]
    out, _ = torch_layer(*ts[:6], M, s)
    (torch.sigmoid(ts[6]) * out * torch.from_numpy(dout)).sum().backward()
    for t, name in zip(ts, ("dq", "dk", "dv", "dtheta", "dbias_u", "dbias_v", "dz")):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)


def test_gate_logit_gradient_by_central_differences():
    rng = _rng(21)
    B, Hg, Wg, H, d, M, s = 1, 8, 8, 1, 8, 4, 2
    q, k, v, z, dout = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(5))
    g = oracle.gated_window_attention_backward(q, k, v, z, dout, M, s)
    flat = z.reshape(-1)
    for i in rng.choice(flat.size, size=12, replace=False):
        keep = flat[i]
        flat[i] = keep + 1e-6
        lp = np.sum(dout * oracle.gated_window_attention(q, k, v, z, M, s))
        flat[i] = keep - 1e-6
        lm = np.sum(dout * oracle.gated_window_attention(q, k, v, z, M, s))
        flat[i] = keep
        assert abs((lp - lm) / 2e-6 - g["dz"].reshape(-1)[i]) < 1e-7


def test_cyclic_schedule():
    assert oracle.cyclic_schedule(6) == [(16, 0), (32, 16), (64, 0), (16, 8), (32, 0), (64, 32)]
    assert oracle.cyclic_schedule(2, (8,)) == [(8, 0), (8, 4)]
