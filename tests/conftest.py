import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU oracle time)")


def pytest_collection_modifyitems(config, items):
    # Run GPU tests in file order but keep the CPU suite first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)
