import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _have_gpu() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped only when the machine has no GPU at all; on a GPU
    # machine a missing or broken HIP library is a failure, never a skip.
    if any("gpu" in item.keywords for item in items) and not _have_gpu():
        skip = pytest.mark.skip(reason="no GPU on this machine")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)
