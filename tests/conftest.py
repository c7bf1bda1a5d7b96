import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # the GPU tests' helpers name their cases past pytest's output capture;
    # CPU-only runs do not depend on that module importing
    try:
        import kda_testlib
    except ImportError:
        return
    kda_testlib.CAPTURE = config.pluginmanager.getplugin("capturemanager")


_GPU_TESTS = set()


def pytest_collection_modifyitems(config, items):
    _GPU_TESTS.update(it.nodeid for it in items if it.get_closest_marker("gpu"))


def pytest_runtest_logstart(nodeid, location):
    # runs outside the test's output capture: each GPU test is named in the
    # output before it starts, whatever the verbosity
    if nodeid in _GPU_TESTS:
        sys.stderr.write("[gpu-test] %s\n" % nodeid)
        sys.stderr.flush()
