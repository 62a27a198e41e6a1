import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a visible GPU; without one they are skipped, so a
    CPU-only run of the whole suite stays green."""
    gpu_items = [i for i in items if "gpu" in i.keywords]
    if not gpu_items:
        return
    import pytest
    import torch
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no GPU visible")
        for item in gpu_items:
            item.add_marker(skip)
