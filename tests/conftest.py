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
    oracle._load()
    return oracle


@pytest.fixture(params=["auto", "256"])
def rows_per_workgroup(request, monkeypatch):
    """Run with the library's own choice of query rows per workgroup (128 for small problems)
    and with 256 forced, so both tile forms of the accumulate kernel meet every case."""
    if request.param != "auto":
        monkeypatch.setenv("Q8A_ROWS_PER_WORKGROUP", request.param)
    return request.param
