import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Write the combine cases checked bit for bit in this session (name and
    element count) to combine_exactness.txt in the folder that the
    MOE_TEST_LOG_DIR environment variable names, when it is set and the
    folder exists."""
    helpers = sys.modules.get("gpu_helpers")
    log = getattr(helpers, "EXACT_LOG", None)
    out_dir = os.environ.get("MOE_TEST_LOG_DIR", "")
    if not log or not out_dir or not os.path.isdir(out_dir):
        return
    total = sum(n for _, n in log)
    with open(os.path.join(out_dir, "combine_exactness.txt"), "w") as f:
        f.write("combine cases whose every output equals the oracle's bits: %d cases, "
                "%d outputs\n" % (len(log), total))
        for what, n in log:
            f.write("%s\t%d\n" % (what, n))
