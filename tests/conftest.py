import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than ~20 s")


def pytest_runtest_logstart(nodeid, location):
    # name the case before it runs, so a run that dies on the GPU says where
    if "gpu" in nodeid or "zz" in nodeid:
        print("\n[start] %s" % nodeid, flush=True)
