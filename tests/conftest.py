import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")



@pytest.fixture(autouse=True)
def _decode_waits_checked(request):
    """After every GPU test: no bounded wait of the decode path gave up in any
    workspace the test's calls used (lowrank_workspace_check)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import rank_decomposed_amd as lr
    lr.watch_workspaces(True)
    try:
        yield
        lr.check_watched_workspaces()
    finally:
        lr.watch_workspaces(False)
