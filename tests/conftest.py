import os
import sys

import pytest
from hypothesis import settings

# property tests draw the same examples on every run, so a pin that fails
# once fails every time
settings.register_profile("pinned", derandomize=True, database=None)
settings.load_profile("pinned")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")
