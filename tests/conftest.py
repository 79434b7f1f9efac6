import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    """The oracle is a small C library; build it once per session if absent."""
    from oracle import build as ob
    if not os.path.exists(ob.LIB):
        ob.build()
