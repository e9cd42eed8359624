"""GPU parity of the row-statistic forward pass and of the backward pass: the HIP path
(through the C ABI) against the float64 oracle on the same seeded inputs.

Bounds.  lse: max|err| <= 1e-2 (the forward pass's bound; lse is a log-sum-exp of logits
that carry the same fp16 operand rounding).  Gradients: relative L2 <= 1e-2 and
max|err| <= 2e-2 * max|ref| per tensor.  The backward pass rounds three more operands than
the forward pass (P to bf16 for dv, dS to fp16 for dq and dk, and dout to bf16), each with
a relative error up to 2^-9 (bf16) or 2^-12 (fp16) per element, and each gradient entry sums
M^2 such products; twice the forward pass's relative-L2 bound covers them.
"""

import numpy as np
import pytest

import oracle
from inputs import qkv, rib_factors, round_bf16, theta_table
from parity_util import errors, note

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 1e-2
GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2e-2


def _setup(B, Hg, Wg, H, M, seed, rope=True, out_f32=True, r=0):
    q, k, v = qkv((B, Hg, Wg, H, 32), seed, "bf16")
    th = theta_table(H, 32, 0.1, seed + 1) if rope else None
    rng = np.random.default_rng(seed + 7)
    dout = rng.normal(size=(B, Hg, Wg, H, 32)).astype(np.float32)
    if not out_f32:
        dout = round_bf16(dout)
    U = V = None
    if r:
        U, V = rib_factors(H, M, r, seed + 2, "bf16")
    return q, k, v, th, dout, U, V


def _gpu(q, k, v, th, dout, M, s, out_f32, U=None, V=None):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    dev = torch.device("cuda:0")
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    odt = torch.float32 if out_f32 else torch.bfloat16
    tq, tk, tv = t(q), t(k), t(v)
    tth = None if th is None else t(th, torch.float32)
    tu = None if U is None else t(U)
    tvb = None if V is None else t(V)
    out, lse = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=odt,
                             return_lse=True)
    plain = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=odt)
    dq, dk, dv, dth, dbu, dbv = wattn.backward(tq, tk, tv, out, t(dout, odt), lse, M=M, shift=s, theta=tth,
                                               bias_u=tu, bias_v=tvb)
    torch.cuda.synchronize()
    f = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)
    return dict(out=f(out), plain=f(plain), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv), dtheta=f(dth),
                dbias_u=f(dbu), dbias_v=f(dbv))


CASES = [
    # label, B, Hg, Wg, H, M, shift, rope, fp32 out
    ("m8_s4", 1, 16, 16, 2, 8, 4, True, True),
    ("m16_s8", 2, 32, 32, 3, 16, 8, True, True),
    ("m32_s16", 1, 64, 64, 2, 32, 16, True, True),
    ("m16_s5_ragged", 1, 48, 32, 2, 16, 5, True, True),
    ("m12_s0_norope", 1, 24, 36, 2, 12, 0, False, True),
    ("m8_s3_bf16_out", 2, 24, 32, 2, 8, 3, True, False),
    ("m4_s1", 1, 8, 12, 2, 4, 1, True, True),
    ("m24_s10", 1, 48, 48, 1, 24, 10, True, True),
    ("m48_s13", 1, 96, 96, 1, 48, 13, True, True),
    ("m32_s16_bf16_out", 1, 64, 64, 1, 32, 16, True, False),
    ("m8_s3_bias", 2, 16, 24, 2, 8, 3, True, True, 16),
    ("m16_s8_bias_bf16_out", 1, 32, 32, 2, 16, 8, True, False, 16),
    ("m24_s0_bias_norope", 2, 48, 48, 1, 24, 0, False, True, 16),
    ("m40_s13_bias", 1, 40, 80, 1, 40, 13, True, True, 16),
    ("m128_s64", 1, 128, 128, 1, 128, 64, True, True),  # the largest window, four wrap regions
    # rank-32 bias factors: a full k = 32 bias operand, two 16-channel blocks of dbias
    ("m8_s3_rank32", 2, 16, 24, 2, 8, 3, True, True, 32),
    ("m16_s8_rank32_bf16_out", 1, 32, 32, 2, 16, 8, True, False, 32),
    ("m32_s16_rank32_norope", 1, 64, 64, 2, 32, 16, False, True, 32),
    ("m40_s13_rank32", 1, 40, 80, 1, 40, 13, True, True, 32),
    # M <= 8: every region fits one workgroup of the fused kernel (as in the M 4 and 8 cases above)
    ("m8_s0_rank32_norope_bf16_out", 1, 24, 16, 3, 8, 0, False, False, 32),
    ("m6_s2_bias", 1, 18, 24, 2, 6, 2, True, True, 16),
    ("m2_s1_bf16_out", 2, 4, 8, 2, 2, 1, True, False),
    # 8 < M < 12: regions beyond one workgroup, the two-kernel path with 2-wave workgroups
    ("m10_s3", 1, 20, 30, 2, 10, 3, True, True),
    ("m11_s5_bias_bf16_out", 1, 22, 22, 2, 11, 5, True, False, 16),
    ("m9_s0_rank32_norope", 2, 18, 27, 1, 9, 0, False, True, 32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    _check_case(case)


def _check_case(case, dout_scale=1.0):
    label, B, Hg, Wg, H, M, s, rope, out_f32 = case[:9]
    r = case[9] if len(case) > 9 else 0
    note(f"backward {label}: B={B} grid={Hg}x{Wg} H={H} M={M} shift={s} rope={rope} fp32_out={out_f32} r={r}")
    q, k, v, th, dout, U, V = _setup(B, Hg, Wg, H, M, 900 + M + s, rope, out_f32, r)
    if dout_scale != 1.0:
        dout = (dout * dout_scale).astype(np.float32)
        if not out_f32:
            dout = round_bf16(dout)
    got = _gpu(q, k, v, th, dout, M, s, out_f32, U, V)
    # the row-statistic forward pass writes the same output as the plain one, bit for bit
    assert np.array_equal(got["out"], got["plain"])
    lse_ref = oracle.window_attention_lse(q, k, M, s, th, U, V)
    lerr, _ = errors(got["lse"], lse_ref)
    note(f"  lse max|err| {lerr:.3e}")
    assert lerr <= LSE_MAX_ABS
    ref = oracle.window_attention_backward(q, k, v, dout, M, s, th, U, V)
    names = ["dq", "dk", "dv"] + (["dtheta"] if rope else []) + (["dbias_u", "dbias_v"] if r else [])
    for name in names:
        mx, rel = errors(got[name], ref[name])
        scale = float(np.max(np.abs(ref[name])))
        note(f"  {name}: max|err| {mx:.3e} (max|ref| {scale:.3e}), rel-L2 {rel:.3e}")
        assert rel <= GRAD_REL_L2, name
        assert mx <= GRAD_MAX_REL * scale, name
    if not rope:
        assert got["dtheta"] is None
    if not r:
        assert got["dbias_u"] is None and got["dbias_v"] is None


# Output gradients far from N(0, 1) (training gradients are often ~1e-4 .. 1e-8 per entry):
# without its power-of-two scale, dS = P (dP - D) rounded to fp16 would fall into the
# subnormal range or flush to zero and dq / dk would lose their accuracy.  The bounds are the
# relative ones above, so the gradients must keep their accuracy at every scale.
SCALE_CASES = [
    ("m32_s16_x1e-6", 1e-6, ("m32_s16", 1, 64, 64, 2, 32, 16, True, True)),
    ("m32_s16_x1e3", 1e3, ("m32_s16", 1, 64, 64, 2, 32, 16, True, True)),
    ("m16_s8_bias_x1e-8", 1e-8, ("m16_s8_bias", 1, 32, 32, 2, 16, 8, True, True, 16)),
    ("m16_s8_rank32_x1e-6", 1e-6, ("m16_s8_rank32", 1, 32, 32, 2, 16, 8, True, True, 32)),
    ("m32_s16_bf16_out_x1e-5", 1e-5, ("m32_s16_bf16_out", 1, 64, 64, 1, 32, 16, True, False)),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_backward_output_gradient_scale(case):
    _check_case(case[2], dout_scale=case[1])


@pytest.mark.parametrize("M,s", [(16, 8), (8, 4)], ids=["m16_two_kernels", "m8_fused"])
def test_backward_region_scales_differ(M, s):
    """Output gradients of very different size in different regions: image 0's are scaled by
    1e-7, image 1's are not.  dk and dv sum over the queries of a key's wrap region, and
    each region takes the gradient scale of its own largest output-gradient entry, so both
    images keep the relative accuracy (one scale for the whole call, set by image 1, would
    round image 0's dS to fp16 zeros and subnormals).  M = 8 runs the fused kernel of small
    regions, M = 16 the query-tile and key-tile kernels."""
    B, Hg, Wg, H = 2, 32, 32, 2
    note(f"backward two scales: B={B} grid={Hg}x{Wg} H={H} M={M} shift={s}")
    q, k, v, th, dout, _, _ = _setup(B, Hg, Wg, H, M, 931)
    dout[0] *= 1e-7
    got = _gpu(q, k, v, th, dout, M, s, True)
    ref = oracle.window_attention_backward(q, k, v, dout, M, s, th)
    for b in range(B):
        for name in ("dq", "dk", "dv"):
            mx, rel = errors(got[name][b], ref[name][b])
            scale = float(np.max(np.abs(ref[name][b])))
            note(f"  image {b} {name}: max|err| {mx:.3e} (max|ref| {scale:.3e}), rel-L2 {rel:.3e}")
            assert rel <= GRAD_REL_L2, (b, name)
            assert mx <= GRAD_MAX_REL * scale, (b, name)


def test_backward_single_token_windows():
    """M = 1: every window holds one token, so P = 1, out = v and dS = P (dP - D) = 0 exactly:
    dq, dk and dtheta are zero and dv is dout.  The kernels compute D from the same bf16 dO as
    dP, so dS vanishes up to the fp32 rounding of the two sums."""
    B, Hg, Wg, H, M, s = 1, 4, 6, 2, 1, 0
    note(f"backward single-token windows: B={B} grid={Hg}x{Wg} H={H} M={M}")
    q, k, v, th, dout, _, _ = _setup(B, Hg, Wg, H, M, 955)
    got = _gpu(q, k, v, th, dout, M, s, True)
    ref = oracle.window_attention_backward(q, k, v, dout, M, s, th)
    for name in ("dq", "dk", "dtheta"):
        assert float(np.max(np.abs(ref[name]))) < 1e-12, name
        mx = float(np.max(np.abs(got[name])))
        note(f"  {name}: max|got| {mx:.3e}")
        assert mx <= 1e-4, name
    mx, rel = errors(got["dv"], ref["dv"])
    note(f"  dv: max|err| {mx:.3e}, rel-L2 {rel:.3e}")
    assert rel <= GRAD_REL_L2


def test_backward_scratch_contract():
    """wattn_backward called through the C ABI with a caller-owned scratch of exactly
    wattn_backward_scratch_bytes, pre-filled with NaN bytes: dq, dk and dv equal the binding's
    (every element of them is written by one thread, with no atomics), so the scratch's
    contents on entry do not matter.  A scratch that is not 16-byte aligned is refused
    (WATTN_ERR_POINTER) before any launch."""
    import ctypes

    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, Wg, H, M, s = 1, 48, 32, 2, 16, 5
    q, k, v, th, dout, _, _ = _setup(B, Hg, Wg, H, M, 977)
    dev = torch.device("cuda:0")
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    tq, tk, tv, tth, tdo = t(q), t(k), t(v), t(th, torch.float32), t(dout, torch.float32)
    out, lse = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, out_dtype=torch.float32, return_lse=True)
    ref = wattn.backward(tq, tk, tv, out, tdo, lse, M=M, shift=s, theta=tth)
    lib = wattn.load_library()
    nbytes = lib.wattn_backward_scratch_bytes(B, H, Hg, Wg, 32)
    rows = B * Hg * Wg * H
    assert nbytes == 4 * ((rows + 3) // 4 * 4 + 33 * rows + 256 * 16 * H)
    scratch = torch.full((nbytes + 64,), 0xFF, dtype=torch.uint8, device=dev)  # NaN bytes
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    dth = torch.empty((H, 16), dtype=torch.float32, device=dev)
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream(dev).cuda_stream)

    def call(scr):
        return lib.wattn_backward(vp(tq.data_ptr()), vp(tk.data_ptr()), vp(tv.data_ptr()), vp(out.data_ptr()),
                                  vp(tdo.data_ptr()), vp(lse.data_ptr()), vp(scr), vp(dq.data_ptr()),
                                  vp(dk.data_ptr()), vp(dv.data_ptr()), vp(dth.data_ptr()), B, H, Hg, Wg, M, s, 32,
                                  vp(tth.data_ptr()), None, None, 0, None, None, 2, stream)  # fp32 out

    assert call(scratch.data_ptr() + 8) == 9  # not 16-byte aligned
    assert call(scratch.data_ptr()) == 0
    torch.cuda.synchronize()
    for name, a, b in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert torch.equal(a, b), name
    # dtheta is accumulated with atomics, so its last bits follow the order of the additions
    r3 = ref[3].cpu().numpy()
    np.testing.assert_allclose(dth.cpu().numpy(), r3, rtol=1e-4, atol=1e-5 * float(np.abs(r3).max()))
