import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    from oracle import build_oracle
    build_oracle.build()
    return oracle.load()


@pytest.fixture
def kda_opts():
    """Set libkda options for one test: kda_opts(name, value) calls
    kda.set_option; every option the test touched is restored afterwards."""
    import gated_delta_rule_104_amd as kda
    saved = {}

    def setopt(name, value):
        if name not in saved:
            saved[name] = kda.get_option(name)
        kda.set_option(name, value)

    yield setopt
    for name, value in saved.items():
        kda.set_option(name, value)
