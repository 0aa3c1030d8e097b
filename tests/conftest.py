import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) when no GPU is visible, so `-m "not gpu"` and plain
    # runs on a CPU-only host behave; on a host with the GPU they run.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture
def hooks():
    """Calls made in the test go through libgdn_hooks.so, the build of the library whose route
    choice honours the GDN_* environment overrides (the release libgdn.so reads no environment)."""
    import gated_deltanet_linear_delta_amd as gdn
    with gdn.test_hooks():
        yield gdn
