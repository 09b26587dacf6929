import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionfinish(session, exitstatus):
    """Write the GPU parity tests' worst errors per case to $GDN_PARITY_JSON."""
    path = os.environ.get("GDN_PARITY_JSON")
    harness = sys.modules.get("gpu_harness")
    if not path or harness is None or not harness.ERRORS:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(harness.ERRORS, f, indent=1, sort_keys=True)
