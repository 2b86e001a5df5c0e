import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long CPU case")


def _ensure(lib_path, build_fn):
    if not os.path.exists(lib_path):
        build_fn()


@pytest.fixture(scope="session", autouse=True)
def _cpu_libs():
    """The oracle and the input generator are plain C; build them once if they are not built yet."""
    from oracle import build as ob
    from synth import build as sb
    _ensure(os.path.join(ROOT, "oracle", "liboracle.so"), ob.build)
    _ensure(os.path.join(ROOT, "synth", "libsynth.so"), sb.build)
    yield
