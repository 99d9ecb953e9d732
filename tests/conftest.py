import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP path through the C ABI")
    config.addinivalue_line("markers", "slow: long CPU test")
    config.addinivalue_line("markers", "nogpu: passes made-up device pointers and relies on the launch failing "
                                       "for want of a GPU; skipped where a GPU is visible")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        # a made-up pointer that passes the host checks would reach a kernel
        skip = pytest.mark.skip(reason="a GPU is visible: the call would launch on made-up pointers")
        for item in items:
            if "nogpu" in item.keywords:
                item.add_marker(skip)
        return
    skip = pytest.mark.skip(reason="no GPU visible in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
