import os
import sys

# Checked mode for every library call the tests make: synchronise after each
# call and raise if a cross-workgroup wait gave up (see set_checked).
os.environ.setdefault("MISCAN_CHECK", "1")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity of the HIP path against the oracle")
