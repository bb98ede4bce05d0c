import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a visible GPU; without one (e.g. a build container) they are skipped.
    With a GPU present they always run, and fail loudly if the library is missing."""
    if not any("gpu" in it.keywords for it in items):
        return
    try:
        import torch
        has_gpu = torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
