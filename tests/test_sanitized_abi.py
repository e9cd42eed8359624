"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

wattn_api.cpp (argument checks, launch planning, dispatch) is built with g++
-fsanitize=address,undefined -fno-sanitize-recover=all into a library whose kernel launchers are
stubs that return an error (tests/asan/launch_stubs.cpp: no device code is built or run), and
tests/test_abi.py runs against it in a child process with the sanitizer runtime preloaded.  Any
out-of-bounds access, use after free, signed overflow or other undefined behaviour on the paths
those tests take aborts the child and fails this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vision_transformer_windowed_window_amd", "csrc")
ROCM = "/opt/rocm"


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the ROCm headers")
def test_abi_checks_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    lib = str(tmp_path / "libwattn_sanitized.so")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(CSRC, "wattn_api.cpp"), os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
             "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", lib]
    res = subprocess.run(build, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               WATTN_TEST_LIBRARY=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout, tail
