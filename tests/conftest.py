import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large-shape case (minutes on the CPU side)")


def pytest_collection_modifyitems(config, items):
    # GPU tests go after the CPU ones so a GPU failure under -x never hides a CPU result.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)
