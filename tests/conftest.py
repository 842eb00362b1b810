"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; all
other tests run on the CPU.
"""
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Test logs (the progress log here, the parity error figures in parity.py)
# go to GQA_TEST_LOG_DIR, by default the folder whose contents come back from
# a remote GPU run.
LOG_DIR = os.environ.get("GQA_TEST_LOG_DIR") or os.path.join(ROOT, "gpurun_out")
PROGRESS = os.path.join(LOG_DIR, "progress.log")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libgqa.so")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build libgqa.so when nothing is built yet (a fresh checkout)."""
    from grouped_query_attention_gemv_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()


@pytest.fixture(autouse=True)
def _progress(request):
    """Name each GPU test in the progress log before it runs, so a run that
    ends abruptly still shows which case was running."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    os.makedirs(os.path.dirname(PROGRESS), exist_ok=True)
    with open(PROGRESS, "a") as f:
        f.write(f"{time.strftime('%H:%M:%S')} start {request.node.nodeid}\n")
    t0 = time.time()
    yield
    with open(PROGRESS, "a") as f:
        f.write(f"{time.strftime('%H:%M:%S')} end   {request.node.nodeid} {time.time() - t0:.1f}s\n")
