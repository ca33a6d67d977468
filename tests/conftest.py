import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    config.addinivalue_line("markers", "oracle_pool: uses the forked CPU-oracle workers of tests/oracle_pool.py")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_collection_finish(session):
    """Fork the oracle workers of the full-size parity tests now, before any
    test touches the GPU, when such tests are selected."""
    if any(item.get_closest_marker("oracle_pool") for item in session.items):
        import oracle_pool
        oracle_pool.start()


def pytest_unconfigure(config):
    import sys
    if "oracle_pool" in sys.modules:
        sys.modules["oracle_pool"].stop()
