import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side case")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden


# The oracle's worker processes for whole-layer parity start before any test
# initialises the GPU, and only when a selected test asks for them.
_ORACLE_POOL = None


@pytest.hookimpl(trylast=True)     # after marker selection has deselected items
def pytest_collection_modifyitems(session, config, items):
    global _ORACLE_POOL
    if any("oracle_pool" in getattr(item, "fixturenames", ()) for item in items):
        from oracle.parallel import OraclePool
        _ORACLE_POOL = OraclePool()


def pytest_sessionfinish(session, exitstatus):
    global _ORACLE_POOL
    if _ORACLE_POOL is not None:
        _ORACLE_POOL.close()
        _ORACLE_POOL = None


@pytest.fixture
def oracle_pool():
    if _ORACLE_POOL is None:
        pytest.skip("oracle worker pool not started")
    return _ORACLE_POOL

