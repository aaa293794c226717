import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionfinish(session, exitstatus):
    """With MOE_PARITY_MARGINS=<file>, write every parity comparison of the
    session (test, tensor, achieved max-rel, bound) there as JSON."""
    path = os.environ.get("MOE_PARITY_MARGINS")
    mod = sys.modules.get("gpu_helpers")
    if not path or mod is None:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(mod.MARGINS, f, indent=1)
