import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle runs")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a CPU-only machine they are
    # deselected by -m "not gpu" and skipped if selected anyway.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
