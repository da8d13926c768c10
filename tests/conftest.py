import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    from tests import gpu_util
    gpu_util.PYTEST_CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
