import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Any test module named test_gpu_* or marked gpu requires the device.
    for item in items:
        if "gpu" in item.keywords:
            continue
        if os.path.basename(str(item.fspath)).startswith("test_gpu_"):
            item.add_marker(pytest.mark.gpu)
