import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running parity case at full workload size")
    config.addinivalue_line("markers", "wait_timeout_path: exercises the give-up path of the bounded waits on purpose")


@pytest.fixture(scope="session")
def oracle_c():
    """The C oracle, built on first use if the shared object is missing."""
    from oracle import kda_ref
    if not os.path.exists(kda_ref.LIB_PATH):
        from oracle import build as obuild
        obuild.build()
    return kda_ref.load_c()


@pytest.fixture(autouse=True)
def device_status_clear(request):
    """After every GPU test: no bounded wait of a library kernel gave up while it ran
    (kda_device_check; a give-up means the outputs of that call were not valid)."""
    yield
    if request.node.get_closest_marker("gpu") is None or request.node.get_closest_marker("wait_timeout_path"):
        return
    import torch

    if not torch.cuda.is_available():
        return
    import gated_delta_rule_chunk_amd as kda

    kda.device_check()
