import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    gpu_items = [i for i in items if "gpu" in i.keywords]
    if not gpu_items:
        return
    import torch
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no HIP device on this host")
        for i in gpu_items:
            i.add_marker(skip)
