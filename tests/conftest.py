import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """With DFLASH_PARITY_MARGINS=<path>, write the float-parity margins of the
    session there (markdown)."""
    path = os.environ.get("DFLASH_PARITY_MARGINS")
    if not path:
        return
    try:
        from tests import gpu_util
    except Exception:
        return
    if gpu_util.MARGINS:
        gpu_util.write_margins(path, ["python"] + sys.argv)
