"""wattn_backward_noalloc through the C ABI against wattn_backward with a caller-owned scratch,
on the same inputs: dq, dk and dv bit for bit (every element is written by one thread, with
no atomics); dtheta and the bias gradients, which are accumulated with atomics in an order
that can differ between calls, to 1e-5 of their largest entry (the tolerance of the caller-
scratch contract test for the same reason).  Two calls in a row, the second on a smaller
problem, so that the library-held scratch is reused with the first call's contents left in
it; the second problem carries the rank-16 bias."""

import ctypes

import numpy as np
import pytest

from inputs import qkv, rib_factors, theta_table
from parity_util import note

pytestmark = pytest.mark.gpu


def _case(B, Hg, Wg, H, M, s, seed, r):
    import torch

    import vision_transformer_windowed_window_amd as wattn

    dev = torch.device("cuda:0")
    q, k, v = qkv((B, Hg, Wg, H, 32), seed, "bf16")
    th = theta_table(H, 32, 0.1, seed + 1)
    dout = np.random.default_rng(seed + 7).normal(size=q.shape).astype(np.float32)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    tq, tk, tv, tth, tdo = t(q), t(k), t(v), t(th, torch.float32), t(dout, torch.float32)
    tu = tvb = None
    if r:
        U, V = rib_factors(H, M, r, seed + 2, "bf16")
        tu, tvb = t(U), t(V)
    out, lse = wattn.forward(tq, tk, tv, M=M, shift=s, theta=tth, bias_u=tu, bias_v=tvb, out_dtype=torch.float32,
                             return_lse=True)
    lib = wattn.load_library()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream(dev).cuda_stream)
    p = lambda x: vp(None if x is None else x.data_ptr())

    def outputs():
        f32 = dict(dtype=torch.float32, device=dev)
        o = [torch.empty(q.shape, **f32) for _ in range(3)] + [torch.empty((H, 16), **f32)]
        o += [torch.empty(tu.shape, **f32), torch.empty(tvb.shape, **f32)] if r else [None, None]
        return o

    ref = outputs()
    scratch = torch.empty(lib.wattn_backward_scratch_bytes(B, H, Hg, Wg, 32), dtype=torch.uint8, device=dev)
    st = lib.wattn_backward(p(tq), p(tk), p(tv), p(out), p(tdo), p(lse), p(scratch), p(ref[0]), p(ref[1]),
                            p(ref[2]), p(ref[3]), B, H, Hg, Wg, M, s, 32, p(tth), p(tu), p(tvb), r, p(ref[4]),
                            p(ref[5]), 2, stream)
    assert st == 0
    got = outputs()
    st = lib.wattn_backward_noalloc(p(tq), p(tk), p(tv), p(out), p(tdo), p(lse), p(got[0]), p(got[1]), p(got[2]),
                                    p(got[3]), B, H, Hg, Wg, M, s, 32, p(tth), p(tu), p(tvb), r, p(got[4]),
                                    p(got[5]), 2, stream)
    assert st == 0
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert torch.equal(a, b), name
    for name, a, b in zip(("dtheta", "dbias_u", "dbias_v"), got[3:], ref[3:]):
        if a is None:
            continue
        err = float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
        note(f"  {name}: max|diff| / max|ref| {err:.2e}")
        assert err <= 1e-5, name


def test_noalloc_matches_caller_scratch_twice():
    note("no-alloc backward: 2 x 64 x 64, 3 heads, M = 32, shift 16 (24576 query rows), then a smaller call")
    _case(2, 64, 64, 3, 32, 16, 1401, 0)
    note("no-alloc backward: 1 x 32 x 48, 2 heads, M = 16, shift 5, rank-16 bias (3072 query rows)")
    _case(1, 32, 48, 2, 16, 5, 1402, 16)


def test_noalloc_fused_small_windows():
    """M = 8: the fused small-region kernel, which takes only the angle-gradient copies from the
    scratch, with the library-held array left as the calls above (or a first call) left it."""
    note("no-alloc backward: 2 x 32 x 32, 3 heads, M = 8, shift 4, rank-32 bias (6144 query rows)")
    _case(2, 32, 32, 3, 8, 4, 1403, 32)
