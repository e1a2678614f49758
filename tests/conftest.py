import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library through the C ABI)")
    config.addinivalue_line("markers", "slow: long CPU check")


@pytest.fixture(scope="session")
def root():
    return ROOT
