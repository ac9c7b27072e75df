import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Writes the worst parity errors of this session's GPU comparisons to
    the file ALSPEC_MARGINS names (nothing if unset or nothing compared)."""
    path = os.environ.get("ALSPEC_MARGINS")
    gu = sys.modules.get("gpu_util")
    if not path or gu is None or not gu.MARGINS:
        return
    import json
    with open(path, "w") as f:
        json.dump(gu.MARGINS, f, indent=0)
