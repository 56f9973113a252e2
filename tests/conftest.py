import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU work")
    import gpu_util

    gpu_util.PYTEST_CONFIG = config


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle._load()
    return oracle
