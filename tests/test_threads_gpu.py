"""Concurrent callers: host threads that call the library at the same time, each on its own
stream, get the results of serial calls.

The forward and backward entry points keep no state between calls (the only cache, the
gate-logit launcher's occupancy figure, is an atomic integer), so calls from several host
threads may overlap.  Four threads each run a forward pass and a backward pass on their own
inputs and their own torch stream, several times over; every output must equal, bit for bit,
the same call made alone beforehand (dq, dk and dv are free of atomics; the angle gradient,
whose sums use atomics, is compared to 1e-5 relative).
"""

import threading

import numpy as np
import pytest

from inputs import qkv, theta_table
from parity_util import note

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 5


def _dev(a, dt):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(torch.device("cuda:0"))


def test_threads_on_separate_streams_match_serial_calls():
    import torch

    import vision_transformer_windowed_window_amd as wattn

    B, Hg, Wg, H = 1, 64, 64, 3
    shape = (B, Hg, Wg, H, 32)
    cases = [(32, 16), (8, 4), (16, 0), (32, 0)]  # (M, shift) per thread
    note(f"threads: {THREADS} x {ROUNDS} rounds, cases {cases}")
    th = _dev(theta_table(H, 32, 0.1, 7), torch.float32)
    work = []
    for i, (M, s) in enumerate(cases):
        q, k, v = (_dev(a, torch.bfloat16) for a in qkv(shape, 700 + i, "bf16"))
        rng = np.random.default_rng(710 + i)
        dout = _dev(rng.normal(size=shape).astype(np.float32), torch.float32)
        work.append(dict(M=M, s=s, q=q, k=k, v=v, dout=dout))

    def run(w):
        out, lse = wattn.forward(w["q"], w["k"], w["v"], M=w["M"], shift=w["s"], theta=th, out_dtype=torch.float32,
                                 return_lse=True)
        grads = wattn.backward(w["q"], w["k"], w["v"], out, w["dout"], lse, M=w["M"], shift=w["s"], theta=th)
        return out, grads[:4]

    ref = [run(w) for w in work]  # serial, on the default stream
    torch.cuda.synchronize()

    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(ROUNDS):
                    out, (dq, dk, dv, dth) = run(work[i])
                    stream.synchronize()
                    r_out, (r_dq, r_dk, r_dv, r_dth) = ref[i]
                    for name, a, b in (("out", out, r_out), ("dq", dq, r_dq), ("dk", dk, r_dk), ("dv", dv, r_dv)):
                        if not torch.equal(a, b):
                            errors.append(f"thread {i} {name}: max|diff| {float((a - b).abs().max()):.3e}")
                    rel = float((dth - r_dth).norm() / r_dth.norm())
                    if rel > 1e-5:
                        errors.append(f"thread {i} dtheta: rel {rel:.3e}")
        except Exception as e:  # surfaced by the main thread
            errors.append(f"thread {i}: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, "; ".join(errors[:8])
