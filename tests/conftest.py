import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running parity case at full workload size")


@pytest.fixture(scope="session")
def oracle_c():
    """The C oracle, built on first use if the shared object is missing."""
    from oracle import kda_ref
    if not os.path.exists(kda_ref.LIB_PATH):
        from oracle import build as obuild
        obuild.build()
    return kda_ref.load_c()
