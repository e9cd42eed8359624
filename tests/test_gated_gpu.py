"""GPU parity of the gated local path: block routing (bit-exact list and count) and the
residual correction out += O_local - O_lin-local (through the C ABI) against the float64
oracle on the same seeded inputs.  The one-launch form (each block's workgroups route
themselves by its gate) must give the list form's output bit for bit.

Bounds on the residual R = out - base: max|err| <= 1e-2 and relative L2 <= 5e-3 (the
bf16 bounds of the attention kernel; the expected relative L2 is about 3e-4: the scores are
exact bf16 products, P and v are rounded to fp16, KV enters through a bf16 high + low
split).  Tokens of unselected blocks must come back bit for bit.
"""

import numpy as np
import pytest

import oracle
from inputs import GATED_CONFIGS, block_gate, make_gated_inputs, qkv, round_bf16
from parity_util import BF16_MAX_ABS, BF16_REL_L2, errors, note

pytestmark = pytest.mark.gpu


def _gpu(q, k, v, base, gate, tau, w, eps, out_f32=True, blocks=None, count=None):
    """Both forms of the path on the same inputs: the list form (wattn_select_blocks +
    wattn_local_residual, or a caller-made list) and, given a gate, the one-launch form
    (wattn_gated_local).  Returns (out of the list form, list, count, out of the one-launch form)."""
    import torch

    import vision_transformer_windowed_window_amd as wattn

    dev = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    tq, tk, tv = (t(a, torch.bfloat16) for a in (q, k, v))
    odt = torch.float32 if out_f32 else torch.bfloat16
    out = t(base, odt)
    fused = None
    if blocks is None:
        tg = t(gate, torch.float32)
        blocks, count = wattn.select_blocks(tg, tau)
        fused = wattn.gated_local_path(tq, tk, tv, t(base, odt), tg, tau, w=w, eps=eps)
    else:
        blocks, count = t(blocks, torch.int32), t(count, torch.int32)
    wattn.local_residual(tq, tk, tv, out, blocks, count, w=w, eps=eps)
    torch.cuda.synchronize()
    n = int(count[0].item())
    f64 = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)
    return f64(out), blocks[:n].cpu().numpy(), n, f64(fused)


def _check_residual(got, base, ref, label):
    mx, rel = errors(got - base, ref - base)
    note(f"{label}: residual max|err| {mx:.3e}, rel-L2 {rel:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, label


CASES = [
    # label, B, Hg, Wg, H, w, tau, eps, fp32 out
    ("w8_tau0.7", 2, 32, 48, 3, 8, 0.7, 1e-6, True),
    ("w16_tau0.5", 1, 64, 64, 2, 16, 0.5, 1e-6, True),
    ("w4_tau0.3", 2, 16, 24, 2, 4, 0.3, 1e-6, True),
    ("w12_tau0.6_ragged_keys", 1, 48, 36, 1, 12, 0.6, 1e-6, True),
    ("w8_all_selected_eps0", 1, 16, 32, 2, 8, -1.0, 0.0, True),
    ("w16_eps0.5", 1, 32, 48, 1, 16, 0.4, 0.5, True),
    ("w8_single_block", 1, 8, 8, 3, 8, 0.0, 1e-6, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gated_local_path_matches_oracle(case):
    label, B, Hg, Wg, H, w, tau, eps, out_f32 = case
    note(f"gated {label}: B={B} grid={Hg}x{Wg} H={H} w={w} tau={tau} eps={eps}")
    seed = 700 + w + Hg
    q, k, v = qkv((B, Hg, Wg, H, 32), seed, "bf16")
    base = np.random.default_rng(seed + 1).standard_normal(size=q.shape).astype(np.float32)
    gate = block_gate(B, Hg // w, Wg // w, seed + 2)
    got, blocks, n, fused = _gpu(q, k, v, base, gate, tau, w, eps, out_f32)
    assert np.array_equal(fused, got), "the one-launch form differs from the list form"
    sel = oracle.select_blocks(gate, tau)
    assert n == sel.size and np.array_equal(blocks, sel), "block list"
    ref = oracle.local_residual(q, k, v, base, sel, w, eps)
    _check_residual(got, base, ref, label)
    untouched = ~np.repeat(np.repeat(gate > tau, w, axis=1), w, axis=2)
    assert np.array_equal(got[untouched], base[untouched].astype(np.float64)), "unselected tokens changed"


def test_bf16_output():
    """bf16 out starting from zero: out = bf16(R), within the bounds plus the final rounding."""
    B, Hg, Wg, H, w = 2, 32, 32, 2, 8
    q, k, v = qkv((B, Hg, Wg, H, 32), 811, "bf16")
    gate = block_gate(B, Hg // w, Wg // w, 812)
    base = np.zeros(q.shape, np.float32)
    got, blocks, n, fused = _gpu(q, k, v, base, gate, 0.5, w, 1e-6, out_f32=False)
    assert np.array_equal(fused, got)
    sel = oracle.select_blocks(gate, 0.5)
    assert np.array_equal(blocks, sel)
    ref = oracle.local_residual(q, k, v, base, sel, w, 1e-6)
    mx, rel = errors(got, ref)
    excess = float(np.max(np.abs(got - ref) - np.abs(ref) * 2.0 ** -8))
    note(f"bf16 out: max|err| {mx:.3e}, rel-L2 {rel:.3e}, beyond rounding {excess:.3e}")
    assert excess <= BF16_MAX_ABS and rel <= BF16_REL_L2


def test_nothing_selected_leaves_out_unchanged():
    B, Hg, Wg, H, w = 1, 32, 32, 3, 8
    q, k, v = qkv((B, Hg, Wg, H, 32), 821, "bf16")
    base = np.random.default_rng(822).standard_normal(size=q.shape).astype(np.float32)
    gate = block_gate(B, Hg // w, Wg // w, 823)
    got, _, n, fused = _gpu(q, k, v, base, gate, 1.0, w, 1e-6)
    assert n == 0 and np.array_equal(got, base.astype(np.float64)) and np.array_equal(fused, got)


def test_gate_ties_and_nan_route_like_the_oracle():
    B, Hg, Wg, H, w = 2, 64, 64, 1, 4
    q, k, v = qkv((B, Hg, Wg, H, 32), 831, "bf16")
    gate = block_gate(B, Hg // w, Wg // w, 832).copy()
    gate.reshape(-1)[::7] = 0.5                # ties with tau are not selected
    gate.reshape(-1)[3::11] = np.nan           # NaN never selected
    base = np.zeros(q.shape, np.float32)
    got, blocks, n, fused = _gpu(q, k, v, base, gate, 0.5, w, 1e-6)
    sel = oracle.select_blocks(gate, 0.5)
    assert n == sel.size and np.array_equal(blocks, sel) and np.array_equal(fused, got)
    _check_residual(got, base, oracle.local_residual(q, k, v, base, sel, w, 1e-6), "ties_nan")


def test_caller_list_with_entries_outside_the_grid():
    """A caller-made list: entries outside the grid are skipped and a count above the number
    of blocks is clamped."""
    B, Hg, Wg, H, w = 1, 16, 16, 2, 8      # 4 blocks
    q, k, v = qkv((B, Hg, Wg, H, 32), 841, "bf16")
    base = np.random.default_rng(842).standard_normal(size=q.shape).astype(np.float32)
    lst = np.array([2, 1 << 20, -3, 0], np.int32)
    got, _, _, _ = _gpu(q, k, v, base, None, None, w, 1e-6, blocks=lst, count=np.array([9], np.int32))
    ref = oracle.local_residual(q, k, v, base, [2, 0], w, 1e-6)
    _check_residual(got, base, ref, "caller_list")


@pytest.mark.parametrize("name", sorted(GATED_CONFIGS))
def test_full_size_sampled(name):
    """The benchmark workload at full size: the list bit-exact, every unselected token
    unchanged, and the residual of 24 sampled selected blocks against the oracle."""
    cfg = GATED_CONFIGS[name]
    inp = make_gated_inputs(cfg)
    note(f"full size {name}: {cfg.B}x{cfg.Hg}x{cfg.Wg} H={cfg.H} w={cfg.w} tau={cfg.tau}")
    got, blocks, n, fused = _gpu(inp["q"], inp["k"], inp["v"], inp["base"], inp["gate"], cfg.tau, cfg.w, cfg.eps)
    sel = oracle.select_blocks(inp["gate"], cfg.tau)
    assert n == sel.size and np.array_equal(blocks, sel) and np.array_equal(fused, got)
    note(f"  {n} of {cfg.blocks} blocks selected")
    untouched = ~np.repeat(np.repeat(inp["gate"] > cfg.tau, cfg.w, axis=1), cfg.w, axis=2)
    assert np.array_equal(got[untouched], inp["base"][untouched].astype(np.float64))
    rng = np.random.default_rng(cfg.seed)
    pick = np.concatenate([sel[:2], sel[-2:], rng.choice(sel, size=20, replace=False)])
    nW = (cfg.Hg // cfg.w) * (cfg.Wg // cfg.w)
    g_all, r_all = [], []
    for blk in np.unique(pick):
        b, ys, xs = oracle.window_tokens(inp["q"], int(blk), cfg.w)
        R = oracle.local_residual_window(inp["q"], inp["k"], inp["v"], int(blk), cfg.w, cfg.eps)
        g_all.append(got[b, ys, xs] - inp["base"][b, ys, xs])
        r_all.append(R)
    _check_residual(np.concatenate(g_all), 0.0, np.concatenate(r_all), f"{name} sampled")
    assert nW > 0
