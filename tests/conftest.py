import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


def pytest_collection_modifyitems(config, items):
    # GPU tests need the device; on a CPU-only host they are skipped, not failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _guard_zones(request):
    """GPU tests: the binding allocates out / workspace / debug buffers between
    guard zones, and every zone is checked when the test ends."""
    if "gpu" not in request.keywords:
        yield
        return
    import paged_kv_cache_08_amd.binding as B
    from tests import gpu_helpers as H
    saved = B._alloc
    B._alloc = H.guarded
    try:
        yield
    finally:
        B._alloc = saved
        H.check_guards()
