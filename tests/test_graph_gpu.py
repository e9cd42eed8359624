"""HIP-graph capture of the library's entry points.

The entry points launch kernels on the caller's stream and nothing else: no allocation, no
memset node (the backward pass clears its atomic targets with a fill kernel) and no host
synchronisation.  A caller can therefore record a call into a HIP graph (here
torch.cuda.CUDAGraph around the ctypes calls, which launch on torch's current stream, the
capture stream) and replay it.  Each test records one call on static buffers, then replays the
graph several times with new inputs copied into those buffers, with eager work and
synchronisations between the replays, and compares every replay with an eager call on the same
inputs: bit for bit where the kernels are deterministic (the forward pass, dq, dk, dv, the
block), within 1e-5 relative where atomic additions order the sums (the angle gradient).
"""

import numpy as np
import pytest

from inputs import block_params, qkv, rib_factors, round_bf16, theta_table
from parity_util import note

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _dev(a, dt):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(torch.device("cuda:0"))


def _capture(fn):
    """Run fn once on a side stream (warm-up, as torch asks before a capture), then record it."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def _eager_noise(t):
    """Unrelated eager work between replays: a reduction over a fresh tensor, read on the host."""
    import torch

    return float((t.float() * 0.5 + 1.0).sum().item())


FWD = [
    # B, Hg, Wg, H, M, shift, rope, r
    (2, 32, 32, 3, 8, 4, True, 0),      # 2-wave kernel, wrap regions
    (1, 64, 64, 3, 32, 16, True, 0),    # 8-wave kernel (the headline's form)
    (1, 32, 32, 2, 16, 0, False, 16),   # rank-16 bias without RoPE
]


@pytest.mark.parametrize("case", FWD, ids=[f"M{c[4]}_s{c[5]}_r{c[7]}" for c in FWD])
def test_forward_graph_replays_match_eager(case):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, Wg, H, M, s, rope, r = case
    note(f"graph forward {case}")
    shape = (B, Hg, Wg, H, 32)
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device="cuda:0") for _ in range(3))
    th = _dev(theta_table(H, 32, 0.1, 3), torch.float32) if rope else None
    bu = bv = None
    if r:
        U, V = rib_factors(H, M, r, 4, "bf16")
        bu, bv = _dev(U, torch.bfloat16), _dev(V, torch.bfloat16)
    out = torch.empty(shape, dtype=torch.float32, device="cuda:0")

    def load(seed):
        a, b, c = qkv(shape, seed, "bf16")
        q.copy_(_dev(a, torch.bfloat16))
        k.copy_(_dev(b, torch.bfloat16))
        v.copy_(_dev(c, torch.bfloat16))

    load(100)
    g, _ = _capture(lambda: wattn.forward(q, k, v, M=M, shift=s, theta=th, bias_u=bu, bias_v=bv, out=out))
    for rep in range(REPLAYS):
        load(200 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = wattn.forward(q, k, v, M=M, shift=s, theta=th, bias_u=bu, bias_v=bv, out_dtype=torch.float32)
        _eager_noise(ref)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"replay {rep}: max|diff| {float((got - ref).abs().max()):.3e}"


@pytest.mark.parametrize("M,s", [(8, 4), (32, 16)])
def test_backward_graph_replays_match_eager(M, s):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, Wg, H = 1, 64, 64, 3
    note(f"graph backward M={M} shift={s}")
    shape = (B, Hg, Wg, H, 32)
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device="cuda:0") for _ in range(3))
    dout = torch.empty(shape, dtype=torch.float32, device="cuda:0")
    out = torch.empty(shape, dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hg, Wg, H), dtype=torch.float32, device="cuda:0")
    th = _dev(theta_table(H, 32, 0.1, 5), torch.float32)

    def load(seed):
        a, b, c = qkv(shape, seed, "bf16")
        q.copy_(_dev(a, torch.bfloat16))
        k.copy_(_dev(b, torch.bfloat16))
        v.copy_(_dev(c, torch.bfloat16))
        o, l = wattn.forward(q, k, v, M=M, shift=s, theta=th, out_dtype=torch.float32, return_lse=True)
        out.copy_(o)
        lse.copy_(l)
        rng = np.random.default_rng(seed + 1)
        dout.copy_(_dev(rng.normal(size=shape).astype(np.float32), torch.float32))

    load(300)
    g, static = _capture(lambda: wattn.backward(q, k, v, out, dout, lse, M=M, shift=s, theta=th))
    dq, dk, dv, dth = static[:4]
    for rep in range(REPLAYS):
        load(400 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dq, dk, dv, dth)]
        ref = wattn.backward(q, k, v, out, dout, lse, M=M, shift=s, theta=th)[:4]
        _eager_noise(ref[0])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert torch.equal(a, b), f"replay {rep} {name}: max|diff| {float((a - b).abs().max()):.3e}"
        rel = float((got[3] - ref[3]).norm() / ref[3].norm())
        assert rel <= 1e-5, f"replay {rep} dtheta: rel {rel:.3e}"


def test_swin_block_graph_replays_match_eager():
    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, H, M, s = 2, 64, 3, 32, 16
    C = 32 * H
    note(f"graph block grid {Hg}x{Hg} C={C} M={M} shift={s}")
    P = block_params(C, 51, "bf16")
    tp = {key: _dev(val, torch.bfloat16 if key.startswith("w_") else torch.float32) for key, val in P.items()}
    tp["theta"] = _dev(theta_table(H, 32, 0.1, 52), torch.float32)
    x = torch.empty((B, Hg, Hg, C), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(wattn.swin_block_workspace(B, Hg, Hg, C), dtype=torch.uint8, device="cuda:0")

    def fresh(seed):
        rng = np.random.default_rng(seed)
        return _dev(round_bf16(rng.standard_normal(size=(B, Hg, Hg, C)).astype(np.float32)), torch.bfloat16)

    x.copy_(fresh(500))
    g, _ = _capture(lambda: wattn.swin_block(x, tp, H=H, M=M, shift=s, workspace=ws))
    for rep in range(REPLAYS):
        x0 = fresh(600 + rep)
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()  # in place on x
        torch.cuda.synchronize()
        got = x.clone()
        ref = x0.clone()
        wattn.swin_block(ref, tp, H=H, M=M, shift=s, workspace=ws)
        _eager_noise(ref)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), f"replay {rep}: max|diff| {float((got.float() - ref.float()).abs().max()):.3e}"
