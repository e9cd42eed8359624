"""The product path has no CPU or non-HIP fallback: without the built library every entry point
raises, and host tensors are refused before any computation."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_MISSING = r"""
import torch
import vision_transformer_windowed_window_amd as w
w.library_path = lambda: "/nonexistent/libwattn.so"
q = torch.zeros((1, 8, 8, 1, 32), dtype=torch.bfloat16)
calls = {
    "forward": lambda: w.forward(q, q, q, M=8),
    "backward": lambda: w.backward(q, q, q, q, q, torch.zeros((1, 8, 8, 1)), M=8),
    "pair_count": lambda: w.pair_count(1, 1, 8, 8, 8, 0),
    "linear": lambda: w.linear(torch.zeros((4, 32), dtype=torch.bfloat16), torch.zeros((4, 32), dtype=torch.bfloat16)),
}
for name, fn in calls.items():
    try:
        fn()
    except RuntimeError as e:
        assert "no non-HIP fallback" in str(e), (name, str(e))
    else:
        raise SystemExit(f"{name} returned without the library")
print("all raised")
"""


def test_every_entry_point_raises_without_the_library():
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    res = subprocess.run([sys.executable, "-c", _MISSING], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all raised" in res.stdout


def test_host_tensors_are_refused():
    import torch

    import vision_transformer_windowed_window_amd as w

    if not os.path.exists(w.library_path()):
        pytest.skip("library not built")
    q = torch.zeros((1, 8, 8, 1, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        w.forward(q, q, q, M=8)
