"""The fp16 range contract of the bf16 modes (include/wattn.h, wattn_forward): the rotated,
scaled queries q log2(e) / sqrt(d), the rotated keys k and the bias factors u log2(e) and v
are rounded to fp16 for the score product, so entries must stay below about 1.8e5 (q) and
4.6e4 (k, u, v); beyond that they overflow and the output must be non-finite, never a wrong
finite value.

Each case puts large entries into one rotation pair (or one bias channel) of one operand and
zeroes the matching pair of the other operand, so the large entries contribute nothing to the
logits: the rest of the logits are the usual N(0, 1) ones and the output is an ordinary,
non-degenerate attention output.  Just below the limit the HIP path must match the oracle
within the parity bounds (the large entries are representable); just above it every
output must be non-finite (an fp16 infinity times zero is NaN in the score product).

A rotated pair keeps its norm, and at least one of its two components reaches norm / sqrt(2)
at any angle, so "below" uses pairs whose norm stays below the fp16 limit and "above" pairs
with norm / sqrt(2) beyond it, whatever the RoPE angle.
"""

import numpy as np
import pytest

from inputs import qkv, rib_factors, round_bf16, theta_table
from parity_util import check, note, oracle_full, run_gpu

pytestmark = pytest.mark.gpu

F16_MAX = 65504.0
QSCALE = 1.4426950408889634 / np.sqrt(32.0)  # log2(e) / sqrt(d), folded into q before rounding


def _base(rope: bool, r: int, seed: int):
    B, Hg, Wg, H, M = 1, 16, 16, 2, 8
    q, k, v = qkv((B, Hg, Wg, H, 32), seed, "bf16")
    th = theta_table(H, 32, 0.1, seed + 1) if rope else None
    U = V = None
    if r:
        U, V = rib_factors(H, M, r, seed + 2, "bf16")
    return dict(q=q, k=k, v=v, theta=th, bias_u=U, bias_v=V), M


def _pair(value_norm: float):
    """Both components of a pair at norm / sqrt(2), rounded to bf16."""
    c = np.float32(value_norm / np.sqrt(2.0))
    return round_bf16(np.array([c, -c], dtype=np.float32))


# operand, limit on the stored component (before the fold for q and u), factor of the case
CASES = [
    ("q_below", "q", F16_MAX / QSCALE, 0.9),
    ("q_above", "q", F16_MAX / QSCALE, 1.6),
    ("k_below", "k", F16_MAX, 0.9),
    ("k_above", "k", F16_MAX, 1.6),
    ("u_below", "u", F16_MAX / 1.4426950408889634, 0.9),
    ("u_above", "u", F16_MAX / 1.4426950408889634, 1.3),
    ("v_below", "v", F16_MAX, 0.9),
    ("v_above", "v", F16_MAX, 1.3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp16_range_contract(case):
    label, operand, limit, factor = case
    bias = operand in ("u", "v")
    inp, M = _base(rope=not bias, r=16 if bias else 0, seed=1234)
    shift = 0 if bias else 4
    if operand == "q":
        inp["q"][..., 0:2] = _pair(factor * limit)  # large pair 0 of every query ...
        inp["k"][..., 0:2] = 0.0                    # ... against zero keys in that pair
    elif operand == "k":
        inp["k"][..., 2:4] = _pair(factor * limit)
        inp["q"][..., 2:4] = 0.0
    elif operand == "u":  # bias channels: no rotation, one channel suffices
        inp["bias_u"][..., 0] = round_bf16(np.full(inp["bias_u"].shape[:-1], factor * limit, np.float32))
        inp["bias_v"][..., 0] = 0.0
    else:
        inp["bias_v"][..., 1] = round_bf16(np.full(inp["bias_v"].shape[:-1], factor * limit, np.float32))
        inp["bias_u"][..., 1] = 0.0
    note(f"{label}: largest {operand} component {factor * limit / (np.sqrt(2.0) if operand in 'qk' else 1):.4g}")
    got = run_gpu(inp, "bf16", M, shift)
    if factor < 1.0:
        check(got, oracle_full(inp, M, shift), "bf16", label)
    else:
        # beyond the fp16 range: every output non-finite, none a finite wrong value
        assert not np.isfinite(got).any(), f"{label}: {np.isfinite(got).sum()} finite outputs"
