import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU work (oracle at full size)")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """With HD_SFA_MARGINS_OUT set, write every checked tensor's worst error
    against the floating-point bar (tests/_check.RECORD) to that JSON file."""
    path = os.environ.get("HD_SFA_MARGINS_OUT")
    if not path:
        return
    import json
    from tests import _check
    rows = [{"what": w, "max_abs_err": e, "max_abs_ref": r, "worst_err_over_maxabs_allowance": q,
             "worst_err_over_base_allowance": b}
            for (w, e, r, q, b) in _check.RECORD]
    with open(path, "w") as f:
        json.dump(rows, f, indent=1)
