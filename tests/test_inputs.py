"""Seeded input generators: determinism, bf16 rounding, theta and bias-factor shapes."""

import hashlib

import numpy as np
import torch

from inputs import CONFIGS, make_inputs, omega_schedule, rib_factors, round_bf16, theta_table


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-42], dtype=np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = round_bf16(x)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(round_bf16(np.array([np.nan], dtype=np.float32)))[0]


def test_generators_are_deterministic():
    cfg = CONFIGS["tiny_fp32"]
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for key in ("q", "k", "v", "theta"):
        np.testing.assert_array_equal(a[key], b[key])
    U1, V1 = rib_factors(6, 8, 16, 3005)
    U2, V2 = rib_factors(6, 8, 16, 3005)
    np.testing.assert_array_equal(U1, U2)
    np.testing.assert_array_equal(V1, V2)
    h = hashlib.sha256(U1.tobytes() + V1.tobytes()).hexdigest()
    assert len(h) == 64


def test_bf16_workload_values_are_bf16_exact():
    cfg = CONFIGS["swin_t_m8"]
    inp = make_inputs(cfg, batch=1)
    for key in ("q", "k", "v"):
        x = inp[key]
        np.testing.assert_array_equal(round_bf16(x), x)
    assert inp["q"].shape == (1, 64, 64, 3, 32)


def test_theta_schedule():
    w = omega_schedule(2, 32, shared=True)
    np.testing.assert_allclose(np.exp(w[0]), 10000.0 ** (-np.arange(8) / 8.0), rtol=1e-12)
    th = theta_table(3, 32, 0.0, 0, shared=True)
    assert th.shape == (3, 16) and th.dtype == np.float32
    np.testing.assert_array_equal(th[:, :8], th[:, 8:])
    tu = theta_table(3, 32, 0.0, 0, shared=False)
    np.testing.assert_allclose(tu[0], 10000.0 ** (-np.arange(16) / 16.0), rtol=1e-6)
    tn = theta_table(3, 32, 0.1, 7, shared=True)
    assert not np.allclose(tn, th)
    np.testing.assert_array_equal(tn[:, :8], tn[:, 8:])


def test_rib_factor_shapes_and_scale():
    U, V = rib_factors(6, 96, 16, 3005)
    assert U.shape == (6, 96 * 96, 16) and V.shape == U.shape
    assert 0.01 < float(np.std(U)) < 5.0
    np.testing.assert_array_equal(round_bf16(U), U)
