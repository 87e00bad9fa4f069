"""pytest configuration: the `gpu` marker and shared fixtures.

CPU tests (-m "not gpu") pin the oracle and the host-side logic; GPU tests
(-m gpu) compare the HIP library with the oracle through the C ABI.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def mm(dev):
    import moe_matvec_amd
    moe_matvec_amd.lib()  # raises if the library is not built: no fallback
    return moe_matvec_amd


@pytest.fixture
def path(mm):
    """Force kernel variants (moe_matvec_testing.h) for one test:
    path(NAME=value, ...); every switch returns to automatic afterwards."""
    def setp(**kw):
        for name, value in kw.items():
            mm.set_path(name, value)
    yield setp
    for name in mm.PATH:
        mm.set_path(name, 0)
