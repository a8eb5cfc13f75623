import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-only check, opt in with BQI_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("BQI_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow exhaustive check; set BQI_SLOW=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)
