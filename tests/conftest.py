import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_host_libs():
    """The oracle and the input generator are plain host C; build them here if
    they are missing so a fresh checkout can run the CPU suite."""
    from oracle import build as ob
    from synth import build as sb
    if not os.path.exists(os.path.join(ROOT, "oracle", "libmoe_oracle.so")):
        ob.build()
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        sb.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


@pytest.fixture(scope="session")
def synth_mod():
    import synth
    return synth
