import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # every decode / append / merge call made through the binding first checks
    # the device-side contract (context lengths, positions, block ids, append
    # targets) on the host; tests that breach it on purpose turn this off
    os.environ.setdefault("MLA_CHECK_CONTRACT", "1")
