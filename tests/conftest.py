import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture
def tuning(monkeypatch):
    """Run this test on the test build of the library (libnormfuse_tuning.so:
    the same kernels, with host code that also reads the NORMFUSE_* tuning
    overrides); returns the monkeypatch fixture, whose setenv sets them."""
    import normalization_ln_fwd_amd as nf
    monkeypatch.setattr(nf, "_lib", nf.load(nf.TUNING_LIB))
    return monkeypatch
