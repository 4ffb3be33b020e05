import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size inputs)")


def pytest_collection_modifyitems(config, items):
    # Run GPU tests in a stable order: probes/ABI first, full-size next to last,
    # the no-allocation entry point's test last (it shares a device array that
    # the library keeps until the process ends)
    def key(item):
        name = item.nodeid
        return (3 if "no_alloc" in name else 2 if "fullsize" in name else 1 if item.get_closest_marker("gpu") else 0)
    items.sort(key=key)
