import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With SDM_PARITY_REPORT set, write the near-tie accounting of every
    labelled slot comparison of the session (tests/parity.py) as JSON."""
    path = os.environ.get("SDM_PARITY_REPORT")
    if not path:
        return
    import json
    import parity
    if parity.REPORT:
        with open(path, "w") as f:
            json.dump({"tolerance": "near tie: S_k - S_k+1 < 1e-6 max(1, |S_k|), every differing slot within "
                                    "that of S_k; literal: gap < 1e-6",
                       "checks": parity.REPORT}, f, indent=1)
