import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: large host-side work (full-size cases)")


def pytest_collection_modifyitems(config, items):
    # A GPU test on a machine without a GPU is an error, not a skip, unless the run
    # deselected GPU tests with -m "not gpu".
    pass
