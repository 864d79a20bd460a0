import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU)")


@pytest.hookimpl(trylast=True)
def pytest_collection_modifyitems(config, items):
    # (after -m and -k have deselected) The host-sanitizer build takes
    # minutes: start it now, so that it runs beside the other tests rather
    # than after them.
    if any(os.path.basename(str(it.fspath)) == "test_zy_host_sanitizers.py" for it in items):
        from test_zy_host_sanitizers import start_build
        start_build()
    # A GPU test on a machine without a GPU is skipped, not failed.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
