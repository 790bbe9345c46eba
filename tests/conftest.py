import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # a fresh checkout has no library yet: build it once (hipcc cross-compiles without a GPU)
    from long_context_exact_ring_amd.build import build_if_missing
    build_if_missing(verbose=False)
