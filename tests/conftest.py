import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes on the CPU side)")
    config.addinivalue_line("markers", "host_lib: uses only libpa's host C++ (allocator, planner, memory "
                                       "simulator, slot checker); also run against the sanitized host build")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; say so instead of failing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
