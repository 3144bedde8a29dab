import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (minutes on CPU)")


_INPUT_CACHE = {}


@pytest.fixture(scope="session")
def config_inputs():
    """Seeded inputs of the five workloads, generated once per session."""
    import workloads

    def get(i):
        if i not in _INPUT_CACHE:
            _INPUT_CACHE[i] = workloads.make_inputs(workloads.workload(i), seed=0)
        return _INPUT_CACHE[i]
    return get
