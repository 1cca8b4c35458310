import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Every forward and backward call the tests make through the binding reads the
# workspace's device error word afterwards and raises if a kernel flagged an
# inconsistency (the binding reads this when it is imported).
os.environ.setdefault("MRA_CHECK_DEVICE_ERRORS", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")
