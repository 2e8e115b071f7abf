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


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_makereport(item, call):
    """Once a failing test's report is written, drop the local variables of
    its traceback's frames: pytest keeps the exception until the session
    ends, and a GPU test's frames hold device tensors and models of tens of
    GiB that later tests in the same process would otherwise not get."""
    outcome = yield
    rep = outcome.get_result()
    if call.excinfo is not None and rep.longrepr is not None:
        import traceback
        try:
            traceback.clear_frames(call.excinfo.tb)
        except Exception:
            pass


def pytest_runtest_teardown(item, nextitem):
    if "gpu" in item.keywords:
        import gc
        gc.collect()
        try:
            import torch
            if torch.cuda.is_available():
                torch.cuda.empty_cache()
        except Exception:
            pass
