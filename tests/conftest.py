import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (runs through the C ABI)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionstart(session):
    # A fresh checkout has no libselattn.so: build it once (hipcc cross-compiles
    # for gfx950 without a GPU). A library that is already built is used as is.
    lib = os.path.join(ROOT, "sparse_top_selection_amd", "libselattn.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_selattn_build", os.path.join(ROOT, "sparse_top_selection_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
