"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's own formula: each compares it with a worked
example, an identity, a library routine (torch's scaled_dot_product_attention on the
CPU in float64), an independent brute force in original image coordinates, or a
second formulation (Swin-style roll + partition + label mask).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from inputs import rib_factors, theta_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------ RoPE


def test_rope_convention_golden():
    """First half of d rotates with the row (y), second half with the column (x)."""
    for case in _load("rope_convention.json")["cases"]:
        th = np.array(case["theta"])
        x = np.array(case["x"], dtype=np.float64)[None, :]
        ang = oracle.rope_angles(th, np.array([case["row"]]), np.array([case["col"]]))
        got = oracle.rope_rotate(x, ang)[0]
        np.testing.assert_allclose(got, case["expected"], atol=1e-12)


def test_rope_relative_identity():
    """<R(p) q, R(p') k> = <q, R(p' - p) k> for arbitrary positions and frequencies."""
    rng = _rng(1)
    for _ in range(50):
        d = 32
        th = np.exp(rng.normal(-1.0, 1.0, size=d // 2))
        q = rng.normal(size=d)
        k = rng.normal(size=d)
        p = rng.integers(-64, 64, size=2)
        pp = rng.integers(-64, 64, size=2)
        rq = oracle.rope_rotate(q[None], oracle.rope_angles(th, p[:1], p[1:]))[0]
        rk = oracle.rope_rotate(k[None], oracle.rope_angles(th, pp[:1], pp[1:]))[0]
        dk = oracle.rope_rotate(k[None], oracle.rope_angles(th, pp[:1] - p[:1], pp[1:] - p[1:]))[0]
        assert abs(rq @ rk - q @ dk) < 1e-11


def test_rope_preserves_norm_and_theta_zero_is_identity():
    rng = _rng(2)
    th = np.exp(rng.normal(size=16))
    x = rng.normal(size=(20, 32))
    r = rng.integers(0, 96, size=20)
    c = rng.integers(0, 96, size=20)
    rx = oracle.rope_rotate(x, oracle.rope_angles(th, r, c))
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(oracle.rope_rotate(x, oracle.rope_angles(np.zeros(16), r, c)), x)


def test_logits_invariant_to_coordinate_offset():
    """Only displacements matter, so shifting every coordinate leaves the logits unchanged."""
    rng = _rng(3)
    M = 8
    qw = rng.normal(size=(M * M, 32))
    kw = rng.normal(size=(M * M, 32))
    th = theta_table(1, 32, 0.1, 5)[0]
    r, c = oracle.local_coords(M)
    a = oracle.window_logits(qw, kw, r, c, th)
    b = oracle.window_logits(qw, kw, r + 17, c - 5, th)
    np.testing.assert_allclose(a, b, atol=1e-11)


def test_logits_take_one_value_per_displacement_3969_at_m32():
    """With the same content at every token, RoPE logits are a function of the displacement
    only, and take exactly as many values as Swin's table has entries (3969 at M = 32)."""
    g = _load("rpb_offsets.json")
    M = g["M"]
    rng = _rng(4)
    th = theta_table(1, 32, 0.1, 6)[0].astype(np.float64)
    r, c = oracle.local_coords(M)
    q0 = rng.normal(size=32)
    k0 = rng.normal(size=32)
    S = oracle.window_logits(np.tile(q0, (M * M, 1)), np.tile(k0, (M * M, 1)), r, c, th)
    dy = r[None, :] - r[:, None]
    dx = c[None, :] - c[:, None]
    key = (dy + M - 1) * (2 * M - 1) + (dx + M - 1)
    groups = {}
    for kk, s in zip(key.ravel(), S.ravel()):
        groups.setdefault(int(kk), []).append(s)
    assert len(groups) == g["entries_per_head"]
    spread = max(max(v) - min(v) for v in groups.values())
    assert spread < 1e-10
    reps = np.array(sorted(v[0] for v in groups.values()))
    assert np.min(np.diff(reps)) > 1e-9  # distinct displacements give distinct logits here


# ---------------------------------------------------------------- shift, mask, softmax


def test_region_sizes_golden():
    """Every row of P has exactly (strip rows x strip cols) equal non-zero weights when all
    logits are equal, matching the hand-derived table."""
    g = _load("region_sizes_8x8_m4_s2.json")
    Hg, Wg, M, s = g["Hg"], g["Wg"], g["M"], g["shift"]
    rf = g["row_factor_by_original_row"]
    cf = g["col_factor_by_original_col"]
    q = np.zeros((1, Hg, Wg, 1, 8))
    k = _rng(5).normal(size=q.shape)
    seen = 0
    for wy in range(Hg // M):
        for wx in range(Wg // M):
            P, y, x = oracle.window_weights(q, k, M, s, 0, wy, wx, 0)
            for i in range(M * M):
                cnt = rf[y[i]] * cf[x[i]]
                nz = P[i][P[i] != 0]
                assert nz.size == cnt
                np.testing.assert_allclose(nz, 1.0 / cnt, rtol=1e-15)
                seen += 1
    assert seen == Hg * Wg


def test_softmax_rows_sum_to_one_and_masked_weights_are_zero():
    rng = _rng(6)
    Hg, Wg, M, s, H, d = 16, 24, 8, 3, 2, 32
    q = rng.normal(size=(1, Hg, Wg, H, d))
    k = rng.normal(size=q.shape)
    th = theta_table(H, d, 0.1, 7)
    U, V = rib_factors(H, M, 4, 8, dtype="fp32")
    for wy, wx in [(0, 0), (Hg // M - 1, 0), (0, Wg // M - 1), (Hg // M - 1, Wg // M - 1)]:
        for h in range(H):
            P, _, _ = oracle.window_weights(q, k, M, s, 0, wy, wx, h, th, U, V)
            np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-13)
            Y, X, _, _, _, _ = oracle.window_token_coords(Hg, Wg, M, s, wy, wx)
            masked = ~np.isfinite(oracle.shift_mask(Y, X, Hg, Wg, M, s))
            assert np.all(P[masked] == 0.0)
            assert np.all(P[~masked] > 0.0)
            if (wy, wx) == (0, 0):
                assert not masked.any()


def test_gather_scatter_is_a_bijection():
    for Hg, Wg, M in [(8, 8, 4), (12, 8, 4), (16, 16, 8)]:
        for s in range(M):
            hit = np.zeros((Hg, Wg), dtype=int)
            for wy in range(Hg // M):
                for wx in range(Wg // M):
                    _, _, y, x, _, _ = oracle.window_token_coords(Hg, Wg, M, s, wy, wx)
                    np.add.at(hit, (y, x), 1)
            assert np.all(hit == 1)


# ------------------------------------------------------------ library reductions (torch)


def _windows(t, M):
    """[B, Hg, Wg, H, d] -> [B, nWy, nWx, H, M*M, d] by plain reshapes (no shift)."""
    B, Hg, Wg, H, d = t.shape
    t = t.reshape(B, Hg // M, M, Wg // M, M, H, d).permute(0, 1, 3, 5, 2, 4, 6)
    return t.reshape(B, Hg // M, Wg // M, H, M * M, d)


def _unwindows(t, Hg, Wg, M):
    B, nWy, nWx, H, N, d = t.shape
    t = t.reshape(B, nWy, nWx, H, M, M, d).permute(0, 1, 4, 2, 5, 3, 6)
    return t.reshape(B, Hg, Wg, H, d)


def test_no_rope_no_bias_no_shift_is_per_window_sdpa():
    rng = _rng(7)
    B, Hg, Wg, M, H, d = 2, 16, 8, 4, 3, 32
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    got = oracle.window_attention(q, k, v, M, 0)
    tq, tk, tv = (_windows(torch.from_numpy(a), M) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    np.testing.assert_allclose(got, _unwindows(ref, Hg, Wg, M).numpy(), atol=1e-12)


def test_single_window_is_global_attention():
    rng = _rng(8)
    B, G, H, d = 1, 8, 2, 16
    q, k, v = (rng.normal(size=(B, G, G, H, d)) for _ in range(3))
    got = oracle.window_attention(q, k, v, G, 0)
    f = lambda a: torch.from_numpy(a).reshape(B, G * G, H, d).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(f(q), f(k), f(v))
    np.testing.assert_allclose(got, ref.transpose(1, 2).reshape(B, G, G, H, d).numpy(), atol=1e-12)


def test_folded_bias_equals_concatenated_channels():
    """[q/sqrt(d), u][k, v]^T = q k^T / sqrt(d) + u v^T: attention over the concatenated
    channels (torch SDPA with scale 1) equals the oracle's explicit-bias attention."""
    rng = _rng(9)
    B, Hg, Wg, M, H, d, r = 2, 8, 16, 8, 2, 32, 16
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    U, V = rib_factors(H, M, r, 10, dtype="fp32")
    U = U.astype(np.float64) * 3.0
    V = V.astype(np.float64) * 3.0
    got = oracle.window_attention(q, k, v, M, 0, None, U, V)
    tq, tk, tv = (_windows(torch.from_numpy(a), M) for a in (q, k, v))
    tu = torch.from_numpy(U).expand(B, Hg // M, Wg // M, H, M * M, r)
    tvb = torch.from_numpy(V).expand(B, Hg // M, Wg // M, H, M * M, r)
    qc = torch.cat([tq / math.sqrt(d), tu], dim=-1)
    kc = torch.cat([tk, tvb], dim=-1)
    ref = torch.nn.functional.scaled_dot_product_attention(qc, kc, tv, scale=1.0)
    np.testing.assert_allclose(got, _unwindows(ref, Hg, Wg, M).numpy(), atol=1e-12)
    # and the bias really matters here (guards against a silently dropped term)
    nob = oracle.window_attention(q, k, v, M, 0)
    assert np.max(np.abs(nob - got)) > 1e-2


def test_zero_bias_and_row_constant_bias_are_no_ops():
    rng = _rng(11)
    B, Hg, Wg, M, s, H, d = 1, 8, 8, 4, 2, 2, 8
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    th = theta_table(H, d, 0.1, 12)
    base = oracle.window_attention(q, k, v, M, s, th)
    Z = np.zeros((H, M * M, 3))
    np.testing.assert_allclose(oracle.window_attention(q, k, v, M, s, th, Z, Z), base, atol=1e-14)
    U = np.zeros((H, M * M, 3))
    U[:, :, 0] = rng.normal(size=(H, M * M)) * 5
    Vb = np.zeros((H, M * M, 3))
    Vb[:, :, 0] = 1.0
    np.testing.assert_allclose(oracle.window_attention(q, k, v, M, s, th, U, Vb), base, atol=1e-12)


def test_roll_partition_label_mask_formulation():
    """Second formulation of the shifted layer: roll the whole grid by -s, cut windows by
    reshape, build the region-label image by slicing, mask pairs with different labels,
    run SDPA with the bias added to the mask, merge windows and roll back by +s."""
    rng = _rng(13)
    for (Hg, Wg, M, s) in [(8, 8, 4, 2), (12, 8, 4, 1), (8, 12, 4, 3), (16, 16, 8, 4), (4, 8, 4, 2)]:
        B, H, d, r = 2, 2, 8, 2
        q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
        U = rng.normal(size=(H, M * M, r))
        Vb = rng.normal(size=(H, M * M, r))
        got = oracle.window_attention(q, k, v, M, s, None, U, Vb)

        roll = lambda a: torch.roll(torch.from_numpy(a), shifts=(-s, -s), dims=(1, 2))
        tq, tk, tv = (_windows(roll(a), M) for a in (q, k, v))
        lab = torch.zeros(Hg, Wg)
        cnt = 0
        for hs in (slice(0, Hg - M), slice(Hg - M, Hg - s), slice(Hg - s, Hg)):
            for ws in (slice(0, Wg - M), slice(Wg - M, Wg - s), slice(Wg - s, Wg)):
                lab[hs, ws] = cnt
                cnt += 1
        lw = lab.reshape(Hg // M, M, Wg // M, M).permute(0, 2, 1, 3).reshape(Hg // M, Wg // M, M * M)
        mask = torch.where(lw[..., :, None] == lw[..., None, :], 0.0, float("-inf")).double()
        bias = torch.from_numpy(U) @ torch.from_numpy(Vb).transpose(1, 2)       # [H, N, N]
        am = mask[None, :, :, None] + bias[None, None, None]
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am)
        ref = torch.roll(_unwindows(o, Hg, Wg, M), shifts=(s, s), dims=(1, 2))
        np.testing.assert_allclose(got, ref.numpy(), atol=1e-12)


# -------------------------------------------------------------------------- brute force


def _rot_pair(a, b, phi):
    return a * math.cos(phi) - b * math.sin(phi), a * math.sin(phi) + b * math.cos(phi)


def _brute_force(q, k, v, M, s, theta, U, V):
    """Pure-Python per-token loops in ORIGINAL image coordinates.

    Key set of token (y, x): tokens of the same shifted window (rolled position
    ((y - s) mod Hg, (x - s) mod Wg) // M) that sit on the same side of the wrap seam on
    both axes (the seam separates original rows y < s from rows y >= s, and likewise for
    columns).  The RoPE term uses the displacement form <q, R(p' - p) k>.
    """
    B, Hg, Wg, H, d = q.shape
    out = np.zeros_like(q)
    d4 = d // 4

    def place(y, x):
        Y, X = (y - s) % Hg, (x - s) % Wg
        return (Y // M, X // M), (Y % M, X % M)

    for b in range(B):
        for h in range(H):
            for y in range(Hg):
                for x in range(Wg):
                    win, (ri, ci) = place(y, x)
                    keys = []
                    for yy in range(Hg):
                        for xx in range(Wg):
                            w2, (rj, cj) = place(yy, xx)
                            if w2 != win:
                                continue
                            if (y < s) != (yy < s) or (x < s) != (xx < s):
                                continue
                            kv = list(k[b, yy, xx, h])
                            if theta is not None:
                                for j in range(d // 2):
                                    dp = (rj - ri) if j < d4 else (cj - ci)
                                    kv[2 * j], kv[2 * j + 1] = _rot_pair(kv[2 * j], kv[2 * j + 1], dp * theta[h][j])
                            logit = sum(qa * ka for qa, ka in zip(q[b, y, x, h], kv)) / math.sqrt(d)
                            if U is not None:
                                logit += sum(ua * va for ua, va in zip(U[h][ri * M + ci], V[h][rj * M + cj]))
                            keys.append((logit, v[b, yy, xx, h]))
                    mx = max(lg for lg, _ in keys)
                    ws = [math.exp(lg - mx) for lg, _ in keys]
                    tot = sum(ws)
                    acc = np.zeros(d)
                    for wgt, (_, vv) in zip(ws, keys):
                        acc += wgt * np.asarray(vv)
                    out[b, y, x, h] = acc / tot
    return out


@pytest.mark.parametrize(
    "Hg,Wg,M,d,r",
    [(4, 4, 2, 4, 0), (8, 8, 4, 8, 2), (12, 8, 4, 4, 2), (8, 12, 4, 8, 0), (4, 4, 4, 8, 2), (12, 12, 4, 4, 0)],
)
def test_brute_force_all_shifts(Hg, Wg, M, d, r):
    rng = _rng(100 + Hg * 10 + Wg + M + d + r)
    B, H = 1, 2
    q, k, v = (rng.normal(size=(B, Hg, Wg, H, d)) for _ in range(3))
    theta = np.exp(rng.normal(-0.5, 0.7, size=(H, d // 2)))
    U = V = None
    if r:
        U = rng.normal(size=(H, M * M, r))
        V = rng.normal(size=(H, M * M, r))
    for s in range(M):
        got = oracle.window_attention(q, k, v, M, s, theta, U, V)
        ref = _brute_force(q, k, v, M, s, theta, U, V)
        np.testing.assert_allclose(got, ref, atol=1e-12, err_msg=f"shift={s}")


def test_unmasked_pair_count_closed_form():
    """Pairs with a finite logit: full windows N^2, windows of the last row or column band
    ((M-s)^2 + s^2) * M^2 (two strips), the corner window ((M-s)^2 + s^2)^2 (four blocks)."""
    for (Hg, Wg, M, s) in [(64, 64, 8, 4), (64, 64, 32, 16), (128, 128, 32, 16), (32, 48, 8, 3), (8, 8, 8, 5)]:
        nwy, nwx = Hg // M, Wg // M
        strip = (M - s) ** 2 + s ** 2
        if s == 0:
            expect = nwy * nwx * M ** 4
        else:
            expect = ((nwy - 1) * (nwx - 1) * M ** 4 + (nwy - 1) * strip * M ** 2
                      + (nwx - 1) * strip * M ** 2 + strip * strip)
        assert oracle.unmasked_pairs(1, 1, Hg, Wg, M, s) == expect
