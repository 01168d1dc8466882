import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Build the HIP library and the oracle when they are missing (they are not kept in git).
_LIB = os.path.join(ROOT, "block_scaled_fp8_token_amd", "libfp8bs.so")
_ORC = os.path.join(ROOT, "oracle", "liboracle.so")
if not os.path.exists(_LIB):
    import importlib.util
    _spec = importlib.util.spec_from_file_location("fp8bs_build", os.path.join(ROOT, "block_scaled_fp8_token_amd", "build.py"))
    _hipbuild = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_hipbuild)
    _hipbuild.build()
if not os.path.exists(_ORC):
    import oracle as _oracle
    _oracle.build(force=True)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
