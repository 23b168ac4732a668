import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(autouse=True)
def _gpu_progress_log(request):
    """Before each GPU test, append its id to test_progress.log in the run's output folder (flushed
    to disk), so a run that ends abruptly still names the case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        out = os.path.join(ROOT, "gpurun_out")
        try:
            os.makedirs(out, exist_ok=True)
            with open(os.path.join(out, "test_progress.log"), "a") as f:
                f.write(f"start {request.node.nodeid}\n")
                f.flush()
                os.fsync(f.fileno())
        except OSError:
            pass
        print(f"[gpu] {request.node.nodeid}", flush=True)
    yield
