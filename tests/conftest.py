import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case that takes tens of seconds")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """The generator and the oracle are plain C built with gcc; build them if absent."""
    import oracle
    import synth
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        synth.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
