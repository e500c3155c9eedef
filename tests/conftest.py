import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_logstart(nodeid, location):
    """With KDV_TEST_TRACE set, name each test on stdout (flushed) before it runs, so that a run that ends
    abruptly still says which test it was in."""
    if os.environ.get("KDV_TEST_TRACE"):
        print(f"\n[start] {nodeid}", flush=True)
