import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible: GPU parity tests are skipped, not passed")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(params=[0, 64, 128], ids=["rows-auto", "rows64", "rows128"])
def prefill_rows(request):
    """The prefill GEMM's tile height: chosen per call (0), or the 64-row
    (groups of 128 or 64 k) or 128-row form (groups of 128 k) forced, so that
    every shape runs each form.  Reset to per-call choice afterwards."""
    from block_wise_int4_amd import mnb as m
    m.mnb_debug_prefill_rows(request.param)
    yield request.param
    m.mnb_debug_prefill_rows(0)
