"""Helpers shared by the GPU parity tests: run the HIP path on seeded inputs and compare
with the float64 oracle."""

from __future__ import annotations

import sys

import numpy as np

import oracle

BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5


def note(msg: str) -> None:
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def to_device(inp: dict, dtype: str):
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    out = {}
    for key in ("q", "k", "v", "bias_u", "bias_v"):
        a = inp.get(key)
        out[key] = None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(tdt).to(dev)
    th = inp.get("theta")
    out["theta"] = None if th is None else torch.from_numpy(np.ascontiguousarray(th, dtype=np.float32)).to(dev)
    return out


def run_gpu(inp: dict, dtype: str, M: int, shift: int, out: str = "fp32"):
    """Run the HIP path; bf16 inputs produce an fp32 output unless out == "bf16"."""
    import torch

    import vision_transformer_windowed_window_amd as wattn

    t = to_device(inp, dtype)
    odt = torch.bfloat16 if (dtype == "bf16" and out == "bf16") else torch.float32
    o = wattn.forward(t["q"], t["k"], t["v"], M=M, shift=shift, theta=t["theta"], bias_u=t["bias_u"],
                      bias_v=t["bias_v"], out_dtype=odt)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def check(got: np.ndarray, ref: np.ndarray, dtype: str, label: str = "", out_bf16: bool = False):
    """The parity bounds (bf16: max|err| <= 1e-2 and rel-L2 <= 5e-3; fp32: 1e-5).  With a bf16
    output the final rounding to bf16 (at most 2^-8 |ref|) comes on top of the kernel's error
    and is allowed for on top of the max|err| bound."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    max_abs, rel = errors(got, ref)
    note(f"{label}: max|err| = {max_abs:.3e}, rel-L2 = {rel:.3e}")
    if out_bf16:
        excess = float(np.max(np.abs(got - ref) - np.abs(ref) * 2.0 ** -8))
        note(f"{label}: max(|err| - 2^-8 |ref|) = {excess:.3e}")
        assert excess <= BF16_MAX_ABS, f"{label}: error beyond the bf16 output rounding {excess:.3e}"
        assert rel <= BF16_REL_L2, f"{label}: rel-L2 {rel:.3e} > {BF16_REL_L2}"
    elif dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS, f"{label}: max|err| {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{label}: rel-L2 {rel:.3e} > {BF16_REL_L2}"
    else:
        assert max_abs <= FP32_MAX_ABS, f"{label}: max|err| {max_abs:.3e} > {FP32_MAX_ABS}"
    return max_abs, rel


def oracle_full(inp: dict, M: int, shift: int):
    return oracle.window_attention(inp["q"], inp["k"], inp["v"], M, shift, inp.get("theta"), inp.get("bias_u"),
                                   inp.get("bias_v"))


def oracle_sampled(inp: dict, M: int, shift: int, units):
    """Oracle rows for a list of (b, wy, wx, h) window-heads; returns [(y, x, h, b, rows)]."""
    res = []
    for (b, wy, wx, h) in units:
        o, y, x = oracle.window_head_output(inp["q"], inp["k"], inp["v"], M, shift, b, wy, wx, h, inp.get("theta"),
                                            inp.get("bias_u"), inp.get("bias_v"))
        res.append((b, y, x, h, o))
    return res


def sample_units(B: int, H: int, Hg: int, Wg: int, M: int, count: int, seed: int):
    """Window-heads to check at full size: the four corner windows of the rolled grid (which
    include every wrap-region shape) plus random ones."""
    rng = np.random.default_rng(seed)
    nwy, nwx = Hg // M, Wg // M
    units = []
    corners = [(0, 0), (nwy - 1, 0), (0, nwx - 1), (nwy - 1, nwx - 1)]
    for i, (wy, wx) in enumerate(corners):
        units.append((int(rng.integers(B)) if i else B - 1, wy, wx, i % H))
    while len(units) < count:
        units.append((int(rng.integers(B)), int(rng.integers(nwy)), int(rng.integers(nwx)), int(rng.integers(H))))
    return sorted(set(units))
