import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes on the CPU")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(20261202)


def pytest_sessionstart(session):
    # tests load the built library: rebuild it unless it was built from the
    # current sources (its embedded build id equals the hash of the tree), so a
    # stale library can never run the tests
    from kv_cache_compression_kvtc_amd.build import ensure_current
    ensure_current(log=lambda m: print(m, file=sys.stderr, flush=True))
