import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity tests of the HIP path")


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_makereport(item, call):
    """A GPU test that fails with anything but an assertion (a HIP error, a
    crash surfacing as an exception) stops the session: no further GPU work
    runs after a device-side failure."""
    outcome = yield
    rep = outcome.get_result()
    if rep.when == "call" and rep.failed and "gpu" in item.keywords:
        if call.excinfo is not None and not call.excinfo.errisinstance(AssertionError):
            item.session.shouldstop = "non-assertion failure in a GPU test"
