"""Shared pytest configuration: the `gpu` marker and repository import paths."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    # Containers without a GPU driver node cannot run GPU tests at all; on a GPU machine
    # (/dev/kfd present) they run and fail loudly if the HIP path is not usable.
    if os.path.exists("/dev/kfd"):
        return
    skip = pytest.mark.skip(reason="no AMD GPU driver node (/dev/kfd) on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
