import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _no_wait_ran_out(request):
    """After every GPU test: no bounded wait of any call on a default workspace
    ran out (a run-out means that call's outputs were unspecified, so a test that
    passed on them would prove nothing).  Tests that force run-outs on purpose
    use workspaces of their own."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import decode_mhc_pre_amd as M
    M.check_default_workspaces(clear=True)
