import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only checks, run with Q4_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("Q4_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow exhaustive check; set Q4_SLOW=1")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
