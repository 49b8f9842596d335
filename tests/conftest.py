import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    gpu_present = None
    for item in items:
        if "gpu" in item.keywords:
            if gpu_present is None:
                try:
                    import torch
                    gpu_present = torch.cuda.is_available()
                except Exception:
                    gpu_present = False
            if not gpu_present:
                item.add_marker(pytest.mark.skip(reason="no GPU in this process"))
