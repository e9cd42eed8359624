"""GPU parity of the convolutional gate: the gate-logit convolutions, the attention forward pass
with the sigmoid gate fused into its epilogue, and the gated backward pass (through the C ABI)
against the float64 oracle on the same seeded inputs.

Bounds: gate logits (bf16 output) max(|err| - 2^-8 |ref|) <= 1e-2 and rel-L2 <= 5e-3; the
gated forward pass the attention's bounds; the gated backward pass the backward pass's bounds
(rel-L2 <= 1e-2, max|err| <= 2e-2 max|ref| per tensor, dz included).
"""

import numpy as np
import pytest

import oracle
from inputs import cla_params, qkv, rib_factors, round_bf16, theta_table
from parity_util import check, errors, note

pytestmark = pytest.mark.gpu

GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2e-2


def _dev(a, dt):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(torch.device("cuda:0"))


# The last two have more output rows (B * ceil(Wg / 16) * Hg) than the GPU holds workgroups,
# so each workgroup's run covers several rows and many runs cross from one strip into the next.
@pytest.mark.parametrize("B,Hg,Wg,C,bias", [(1, 8, 8, 32, True), (2, 24, 40, 96, True), (1, 16, 20, 192, False),
                                            (1, 9, 7, 64, True), (1, 32, 32, 256, True), (3, 5, 13, 160, False),
                                            (2, 192, 192, 192, True), (4, 203, 120, 32, False)])
def test_cla_logits_match_oracle(B, Hg, Wg, C, bias):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    note(f"cla logits B={B} grid={Hg}x{Wg} C={C} bias={bias}")
    x = round_bf16(np.random.default_rng(C + Hg).standard_normal(size=(B, Hg, Wg, C)).astype(np.float32))
    w_dw, b_dw, w_pw, b_pw = cla_params(C, 17 + C)
    if not bias:
        b_dw = b_pw = None
    z = wattn.cla_logits(_dev(x, torch.bfloat16), _dev(w_dw, torch.float32), _dev(w_pw, torch.float32),
                         None if b_dw is None else _dev(b_dw, torch.float32),
                         None if b_pw is None else _dev(b_pw, torch.float32))
    torch.cuda.synchronize()
    got = z.float().cpu().numpy().astype(np.float64)
    ref = oracle.cla_gate_logits(x, w_dw, np.zeros(C) if b_dw is None else b_dw, w_pw,
                                 np.zeros(C) if b_pw is None else b_pw)
    check(got, ref, "bf16", f"cla C={C}", out_bf16=True)


def _gated_inputs(B, Hg, Wg, H, M, seed, rope=True, r=0):
    q, k, v = qkv((B, Hg, Wg, H, 32), seed, "bf16")
    th = theta_table(H, 32, 0.1, seed + 1) if rope else None
    U = V = None
    if r:
        U, V = rib_factors(H, M, r, seed + 2, "bf16")
    z = round_bf16((1.5 * np.random.default_rng(seed + 3).standard_normal(size=q.shape)).astype(np.float32))
    return q, k, v, th, U, V, z


CASES = [
    # label, B, Hg, Wg, H, M, shift, rope, r, fp32 out
    ("m8_s4", 2, 16, 24, 3, 8, 4, True, 0, True),
    ("m8_s3_bias_bf16_out", 1, 24, 16, 2, 8, 3, True, 16, False),  # the fused small-region backward
    ("m32_s16", 1, 64, 64, 2, 32, 16, True, 0, True),
    ("m16_bias_norope", 1, 32, 48, 2, 16, 0, False, 16, True),
    ("m16_s5_bf16_out", 1, 48, 32, 2, 16, 5, True, 0, False),
    ("m10_s3_bias", 1, 20, 30, 2, 10, 3, True, 16, True),  # the 2-wave two-kernel backward
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gated_forward_and_backward_match_oracle(case):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    label, B, Hg, Wg, H, M, s, rope, r, out_f32 = case
    note(f"gated attention {label}: B={B} grid={Hg}x{Wg} H={H} M={M} shift={s} rope={rope} r={r}")
    q, k, v, th, U, V, z = _gated_inputs(B, Hg, Wg, H, M, 950 + M + s, rope, r)
    odt = torch.float32 if out_f32 else torch.bfloat16
    tq, tk, tv, tz = (_dev(a, torch.bfloat16) for a in (q, k, v, z))
    tth = None if th is None else _dev(th, torch.float32)
    tu = None if U is None else _dev(U, torch.bfloat16)
    tvb = None if V is None else _dev(V, torch.bfloat16)
    out, lse = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=odt,
                             return_lse=True, gate_z=tz)
    plain, lse0 = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=odt,
                                return_lse=True)
    half = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=odt,
                         gate_z=torch.zeros_like(tz))
    rng = np.random.default_rng(7)
    dout = rng.standard_normal(size=q.shape).astype(np.float32)
    if not out_f32:
        dout = round_bf16(dout)
    grads = wattn.backward(tq, tk, tv, out, _dev(dout, odt), lse, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb,
                           gate_z=tz)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    # the gate leaves the row statistic alone, and a zero logit halves the output exactly
    assert torch.equal(lse, lse0)
    assert torch.equal(half.float(), plain.float() * 0.5)
    ref = oracle.gated_window_attention(q, k, v, z, M, s, th, U, V)
    check(f(out), ref, "bf16", f"gated fwd {label}", out_bf16=not out_f32)
    g_ref = oracle.gated_window_attention_backward(q, k, v, z, dout, M, s, th, U, V)
    names = ["dq", "dk", "dv"] + (["dtheta"] if rope else []) + (["dbias_u", "dbias_v"] if r else [])
    got = dict(zip(["dq", "dk", "dv", "dtheta", "dbias_u", "dbias_v", "dz"], [f(t) for t in grads]))
    for name in names + ["dz"]:
        mx, rel = errors(got[name], g_ref[name])
        scale = float(np.max(np.abs(g_ref[name])))
        note(f"  {name}: max|err| {mx:.3e} (max|ref| {scale:.3e}), rel-L2 {rel:.3e}")
        assert rel <= GRAD_REL_L2 and mx <= GRAD_MAX_REL * scale, name


def test_logits_feed_the_gated_forward_pass():
    """The two kernels in sequence: z = wattn_cla_logits(x) then the gated forward pass, against
    the oracle's z (rounded to bf16 as the kernel stores it) and gated attention."""
    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, Wg, H, M, s = 2, 32, 32, 3, 16, 8
    C = H * 32
    q, k, v = qkv((B, Hg, Wg, H, 32), 971, "bf16")
    x = round_bf16(np.random.default_rng(972).standard_normal(size=(B, Hg, Wg, C)).astype(np.float32))
    w_dw, b_dw, w_pw, b_pw = cla_params(C, 973)
    th = theta_table(H, 32, 0.1, 974)
    tz = wattn.cla_logits(_dev(x, torch.bfloat16), _dev(w_dw, torch.float32), _dev(w_pw, torch.float32),
                          _dev(b_dw, torch.float32), _dev(b_pw, torch.float32))
    out = wattn.forward(_dev(q, torch.bfloat16), _dev(k, torch.bfloat16), _dev(v, torch.bfloat16), M=M, shift=s,
                        theta=_dev(th, torch.float32), out_dtype=torch.float32, gate_z=tz.view(B, Hg, Wg, H, 32))
    torch.cuda.synchronize()
    z_ref = round_bf16(oracle.cla_gate_logits(x, w_dw, b_dw, w_pw, b_pw).astype(np.float32)).reshape(q.shape)
    ref = oracle.gated_window_attention(q, k, v, z_ref, M, s, th)
    check(out.cpu().numpy().astype(np.float64), ref, "bf16", "logits -> gated forward")


def test_cyclic_stack_layers_match_oracle():
    """A reduced stack (one image of 64 x 64 tokens, 2 heads): every layer of the cyclic schedule
    16, 32, 64 with its rank-16 bias and gate, computed as bench.py's stack pass does."""
    import dataclasses

    import torch

    import vision_transformer_windowed_window_amd as wattn
    from inputs import STACK_CONFIGS, make_stack_layer

    cfg = dataclasses.replace(STACK_CONFIGS["sst_cycle_sr"], B=1, Hg=64, Wg=64, H=2,
                              layers=tuple(oracle.cyclic_schedule(6)))
    for l, (M, shift) in enumerate(cfg.layers):
        inp = make_stack_layer(cfg, l)
        d = {key: _dev(inp[key], torch.bfloat16) for key in ("q", "k", "v", "x", "bias_u", "bias_v")}
        d.update({key: _dev(inp[key], torch.float32) for key in ("w_dw", "b_dw", "w_pw", "b_pw")})
        z = wattn.cla_logits(d["x"], d["w_dw"], d["w_pw"], d["b_dw"], d["b_pw"])
        out = wattn.forward(d["q"], d["k"], d["v"], M=M, shift=shift, bias_u=d["bias_u"], bias_v=d["bias_v"],
                            out_dtype=torch.float32, gate_z=z.view(d["q"].shape))
        torch.cuda.synchronize()
        z_ref = round_bf16(oracle.cla_gate_logits(inp["x"], inp["w_dw"], inp["b_dw"], inp["w_pw"],
                                                  inp["b_pw"]).astype(np.float32)).reshape(inp["q"].shape)
        ref = oracle.gated_window_attention(inp["q"], inp["k"], inp["v"], z_ref, M, shift, None, inp["bias_u"],
                                            inp["bias_v"])
        check(out.cpu().numpy().astype(np.float64), ref, "bf16", f"stack layer {l} M={M} shift={shift}")
