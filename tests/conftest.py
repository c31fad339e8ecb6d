import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "fake_pointers: passes fake, never-dereferenced device pointers to check "
                                       "that validation refuses a call before any launch (skipped where a GPU "
                                       "is visible, so a validation regression cannot launch on them)")


def _gpu_visible():
    # counting devices does not initialise the GPU
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    marked = [it for it in items if it.get_closest_marker("fake_pointers")]
    if marked and _gpu_visible():
        skip = pytest.mark.skip(reason="fake device pointers are only passed where no GPU is visible")
        for it in marked:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.build()
    return o
