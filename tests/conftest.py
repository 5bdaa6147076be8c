import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session", autouse=True)
def oracle_workers(request):
    """Fork the oracle's worker pool before the first GPU test runs (no device
    state to inherit), when any selected test uses the GPU."""
    items = getattr(request.session, "items", [])
    if not any(it.get_closest_marker("gpu") for it in items):
        yield None
        return
    from tests import oracle_pool
    pool = oracle_pool.start()
    yield pool
    oracle_pool.stop()
