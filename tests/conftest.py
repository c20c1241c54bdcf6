import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")
    import tests._gpu as g   # progress notes of the GPU tests go through pytest's capture manager
    g.CONFIG = config


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly when they run without a GPU; they are only deselected by -m.
    pass


def pytest_report_header(config):
    return f"repo root: {ROOT}"
