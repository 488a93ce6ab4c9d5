import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(1234)


def _ensure_built():
    """Build the oracle and the HIP library in-tree if a built copy is missing
    (both builds are CPU-only: hipcc cross-compiles for gfx950)."""
    lib = os.path.join(ROOT, "moe_decode_gate_amd", "lib", "libwd.so")
    if not os.path.exists(lib):
        from moe_decode_gate_amd import build as b
        b.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        from oracle import build as ob
        ob.build()


_ensure_built()
