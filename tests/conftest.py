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
    # tests load the built library; build it only when nothing is built yet
    lib = os.path.join(ROOT, "kv_cache_compression_kvtc_amd", "libkvtc.so")
    if not os.path.exists(lib):
        from kv_cache_compression_kvtc_amd.build import build
        build()
