"""Build libwattn.so and the pipe_rates and access_rates programs in-tree with hipcc for gfx950.

Usage: python -m vision_transformer_windowed_window_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwattn.so")
PIPE_RATES = os.path.join(PKG, "pipe_rates")  # instruction-rate probe run by bench.py
ACCESS_RATES = os.path.join(PKG, "access_rates")  # HBM rate of the small-window access pattern
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around each MFMA)
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwattn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    """Compile csrc/ into libwattn.so, pipe_rates and access_rates next to this file; return the library path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="wattn_build_") as tmp:
        kobj = os.path.join(tmp, "wattn_kernels.o")
        gobj = os.path.join(tmp, "wattn_gated.o")
        cobj = os.path.join(tmp, "wattn_cla.o")
        mobj = os.path.join(tmp, "wattn_model.o")
        nobj = os.path.join(tmp, "wattn_noalloc.o")
        aobj = os.path.join(tmp, "wattn_api.o")
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, "wattn_kernels.hip"), "-o", kobj], verbose)
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, "wattn_gated.hip"), "-o", gobj], verbose)
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, "wattn_cla.hip"), "-o", cobj], verbose)
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, "wattn_model.hip"), "-o", mobj], verbose)
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, "wattn_noalloc.hip"), "-o", nobj], verbose)
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
        _run([hipcc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-c",
              os.path.join(CSRC, "wattn_api.cpp"), "-o", aobj], verbose)
        out_tmp = os.path.join(tmp, "libwattn.so")
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", kobj, gobj, cobj, mobj, nobj, aobj, "-o", out_tmp], verbose)
        shutil.move(out_tmp, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
        exe_tmp = os.path.join(tmp, "pipe_rates")
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, os.path.join(CSRC, "pipe_rates.hip"),
              "-o", exe_tmp], verbose)
        shutil.move(exe_tmp, PIPE_RATES + ".tmp")
        os.replace(PIPE_RATES + ".tmp", PIPE_RATES)
        acc_tmp = os.path.join(tmp, "access_rates")
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, os.path.join(CSRC, "access_rates.hip"),
              "-o", acc_tmp], verbose)
        shutil.move(acc_tmp, ACCESS_RATES + ".tmp")
        os.replace(ACCESS_RATES + ".tmp", ACCESS_RATES)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
