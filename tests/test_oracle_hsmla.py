"""Pins of the gated local path's oracle (CPU only).

Each oracle function is checked against something that does not reuse its own code path:
numpy's flatnonzero for the routing, the associative O(N d^2) evaluation order of linear
attention, torch's scaled_dot_product_attention and the already-pinned shifted-window
oracle for the softmax part, closed forms (constant values, zero features), and a
scalar-loop brute force over tokens in original image coordinates.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from inputs import block_gate, round_bf16


def _rng(seed):
    return np.random.default_rng(seed)


# ---- routing ---------------------------------------------------------------------------

def test_select_matches_flatnonzero_with_ties_and_nan():
    g = block_gate(3, 4, 5, 11).copy()
    g[0, 1, 2] = 0.5           # equal to tau: not selected (strict comparison)
    g[2, 3, 4] = np.nan        # never selected
    g[1, 0, 0] = np.nextafter(np.float32(0.5), np.float32(1.0))  # just above
    got = oracle.select_blocks(g, 0.5)
    with np.errstate(invalid="ignore"):
        ref = np.flatnonzero(g.reshape(-1) > np.float32(0.5))
    np.testing.assert_array_equal(got, ref)
    assert 1 * 4 * 5 + 0 in got and (0 * 4 + 1) * 5 + 2 not in got
    assert np.all(np.diff(got) > 0)


@pytest.mark.parametrize("tau,expect", [(-1.0, "all"), (1.0, "none")])
def test_select_all_and_none(tau, expect):
    g = block_gate(2, 3, 3, 12)
    got = oracle.select_blocks(g, tau)
    if expect == "all":
        np.testing.assert_array_equal(got, np.arange(g.size))
    else:
        assert got.size == 0


def test_block_numbering():
    """Block 7 of a 2-image grid of 2 x 3 windows is image 1, window row 0, column 1."""
    assert oracle.block_origin(7, 2, 3, 8) == (1, 0, 8)
    assert oracle.block_origin(5, 2, 3, 4) == (0, 4, 8)
    assert oracle.block_origin(0, 2, 3, 4) == (0, 0, 0)


# ---- linear attention ------------------------------------------------------------------

def test_linear_attention_associative_form():
    """The materialised weights and phi(Q) (phi(K)^T V) / (phi(Q) sum phi(K) + eps) agree."""
    rng = _rng(21)
    q, k, v = (rng.normal(size=(37, 8)) for _ in range(3))
    for eps in (0.0, 1e-6, 0.5):
        got = oracle.relu_linear_attention(q, k, v, eps)
        fq, fk = np.maximum(q, 0), np.maximum(k, 0)
        kv = fk.T @ v                              # [d][d], summed over keys first
        ref = (fq @ kv) / (fq @ fk.sum(axis=0) + eps)[:, None]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_linear_attention_closed_forms():
    rng = _rng(22)
    q, k = rng.normal(size=(10, 8)), rng.normal(size=(12, 8))
    c = rng.normal(size=8)
    # constant values: a convex combination returns the constant (eps = 0)
    np.testing.assert_allclose(oracle.relu_linear_attention(np.abs(q), k, np.tile(c, (12, 1)), 0.0),
                               np.tile(c, (10, 1)), rtol=1e-12, atol=1e-12)
    # a query with no positive channel sees zero weights: output 0 for any eps > 0
    o = oracle.relu_linear_attention(-np.abs(q), k, rng.normal(size=(12, 8)), 1e-6)
    assert np.all(o == 0.0)
    # identical keys give uniform weights: the mean of the values, scaled by S / (S + eps)
    kk = np.tile(np.abs(k[0]), (12, 1))
    vv = rng.normal(size=(12, 8))
    qq = np.abs(q)
    S = (qq @ kk[0])[:, None] * 12
    np.testing.assert_allclose(oracle.relu_linear_attention(qq, kk, vv, 0.25),
                               vv.mean(axis=0)[None, :] * S / (S + 0.25), rtol=1e-12)


def test_global_linear_attention_is_per_image_and_head():
    rng = _rng(23)
    q, k, v = (rng.normal(size=(2, 4, 6, 2, 8)) for _ in range(3))
    got = oracle.global_linear_attention(q, k, v, 1e-6)
    for b in range(2):
        for h in range(2):
            flat = lambda t: t[b, :, :, h].reshape(24, 8)
            fq, fk = np.maximum(flat(q), 0), np.maximum(flat(k), 0)
            ref = (fq @ (fk.T @ flat(v))) / (fq @ fk.sum(axis=0) + 1e-6)[:, None]
            np.testing.assert_allclose(got[b, :, :, h].reshape(24, 8), ref, rtol=1e-12, atol=1e-12)


# ---- softmax part and the residual -----------------------------------------------------

def test_softmax_attention_matches_sdpa():
    rng = _rng(31)
    q, k, v = (rng.normal(size=(64, 32)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None, None] for a in (q, k, v)))[0, 0].numpy()
    np.testing.assert_allclose(oracle.softmax_attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def test_all_blocks_with_nonpositive_keys_is_unshifted_window_attention():
    """With every key channel <= 0 the linear weights vanish (O_lin-local = 0 for eps > 0), so
    selecting every block adds plain unshifted window attention to the base."""
    rng = _rng(32)
    B, Hg, Wg, H, d, w = 2, 8, 12, 2, 8, 4
    q, v, base = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    k = -np.abs(rng.normal(size=(B, Hg, Wg, H, d)))
    nb = B * (Hg // w) * (Wg // w)
    got = oracle.local_residual(q, k, v, base, np.arange(nb), w, 1e-6)
    ref = base + oracle.window_attention(q, k, v, w, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_empty_selection_returns_base():
    rng = _rng(33)
    q, k, v, base = (rng.normal(size=(1, 8, 8, 1, 4)) for _ in range(4))
    out = oracle.gated_local_path(q, k, v, base, np.zeros((1, 2, 2), np.float32), 0.5, 4, 1e-6)
    assert np.array_equal(out, base)


def test_constant_values_give_zero_residual():
    """Both attentions return a constant value vector unchanged (eps = 0, positive features)."""
    rng = _rng(34)
    B, Hg, Wg, H, d, w = 1, 8, 8, 2, 8, 4
    q, k = (np.abs(rng.normal(size=(B, Hg, Wg, H, d))) + 0.1 for _ in range(2))
    v = np.broadcast_to(rng.normal(size=d), (B, Hg, Wg, H, d)).copy()
    base = rng.normal(size=(B, Hg, Wg, H, d))
    got = oracle.local_residual(q, k, v, base, np.arange(4), w, 0.0)
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-12)


def _brute_force(q, k, v, base, gate, tau, w, eps):
    """Per token, in original image coordinates, with scalar loops: a selected token's keys are
    the tokens of the w x w tile containing it."""
    B, Hg, Wg, H, d = q.shape
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out = base.astype(np.float64).copy()
    for b in range(B):
        for y in range(Hg):
            for x in range(Wg):
                if not gate[b, y // w, x // w] > tau:
                    continue
                keys = [(yy, xx) for yy in range(Hg) for xx in range(Wg) if yy // w == y // w and xx // w == x // w]
                for h in range(H):
                    qv = q[b, y, x, h]
                    logits = [sum(qv[c] * k[b, yy, xx, h, c] for c in range(d)) / math.sqrt(d) for yy, xx in keys]
                    mx = max(logits)
                    e = [math.exp(s - mx) for s in logits]
                    lin = [sum(max(qv[c], 0.0) * max(k[b, yy, xx, h, c], 0.0) for c in range(d)) for yy, xx in keys]
                    den = sum(lin) + eps
                    for c in range(d):
                        o_loc = sum(e[j] * v[b, yy, xx, h, c] for j, (yy, xx) in enumerate(keys)) / sum(e)
                        o_lin = sum(lin[j] * v[b, yy, xx, h, c] for j, (yy, xx) in enumerate(keys)) / den
                        out[b, y, x, h, c] += o_loc - o_lin
    return out


@pytest.mark.parametrize("Hg,Wg,w", [(8, 8, 4), (8, 12, 4), (6, 4, 2)])
def test_brute_force_tiny_grids(Hg, Wg, w):
    rng = _rng(40 + Hg + Wg + w)
    B, H, d = 2, 2, 4
    q, k, v = (round_bf16(rng.normal(size=(B, Hg, Wg, H, d)).astype(np.float32)) for _ in range(3))
    base = rng.normal(size=(B, Hg, Wg, H, d))
    gate = block_gate(B, Hg // w, Wg // w, 41)
    got = oracle.gated_local_path(q, k, v, base, gate, 0.4, w, 1e-3)
    ref = _brute_force(q, k, v, base, gate, 0.4, w, 1e-3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the untouched tokens keep the base exactly
    sel = np.repeat(np.repeat(gate > 0.4, w, axis=1), w, axis=2)
    assert np.array_equal(got[~sel], base[~sel])
