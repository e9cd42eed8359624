import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


def pytest_sessionstart(session):
    # tests/test_sanitized_abi.py runs the C-ABI tests against a sanitizer build of the host API
    # (no device code): it names that library here, for the binding to load instead of the
    # in-tree libwattn.so
    path = os.environ.get("WATTN_TEST_LIBRARY")
    if path:
        import vision_transformer_windowed_window_amd as wattn

        wattn.library_path = lambda: path
