import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture
def progress(request):
    """progress(msg): a line written to the terminal at once, past pytest's
    output capture, so that a test running for minutes shows it is alive."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def say(msg):
        if capman is None:
            print(msg, flush=True)
            return
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)

    return say
