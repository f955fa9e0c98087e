import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them loudly rather than erroring on import.
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """With RS_GRAD_REPORT=<path>, write the achieved gradient error ratios of every bf16/fp16
    gradient check (test, tensor, max|err|/RMS, RMS(err)/RMS, bf16 rounding floor)."""
    path = os.environ.get("RS_GRAD_REPORT")
    if not path:
        return
    try:
        from parity_util import GRAD_REPORT
    except Exception:
        return
    import json

    with open(path, "w") as f:
        for row in GRAD_REPORT:
            f.write(json.dumps(row) + "\n")
