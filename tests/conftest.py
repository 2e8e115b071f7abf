import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: long-running parity case")


def _ensure_host_libs():
    """The oracle and the host generator are cheap gcc builds; build them if a
    fresh checkout lacks them."""
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        from synth import build as sb
        sb.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def root():
    return ROOT
