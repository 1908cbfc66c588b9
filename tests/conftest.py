import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_logstart(nodeid, location):
    # name every test on the real stderr before it runs, so a run that dies on the GPU still
    # says which case it was in
    if "gpu" in nodeid or os.environ.get("KDA_TEST_TRACE"):
        sys.__stderr__.write(f"[start] {nodeid}\n")
        sys.__stderr__.flush()


def pytest_runtest_logreport(report):
    # errors a GPU test measured (tests/errlog.py), after its call phase
    if report.when != "call":
        return
    import errlog
    for line in errlog.PENDING:
        sys.__stderr__.write(line + "\n")
    sys.__stderr__.flush()
    errlog.PENDING.clear()


def pytest_collection_modifyitems(config, items):
    gpu_items = [it for it in items if it.get_closest_marker("gpu")]
    if not gpu_items:
        return
    import torch
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no HIP device visible")
        for it in gpu_items:
            it.add_marker(skip)
