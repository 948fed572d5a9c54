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


@pytest.fixture(params=["128", "256", "256k", "64"])
def rows_per_workgroup(request):
    """Run with each tile form of the accumulate kernel forced for more than 64 query rows: 128
    rows per workgroup, 256 rows, 256 rows with every tile's keys split over 8 wavefronts, and
    64 rows with every tile's keys split over wavefront pairs (tests without this fixture run
    the library's own choice).  The form is set in the flags of every state
    gpu_util.new_state describes."""
    import gpu_util
    gpu_util.TILE_FORM[0] = gpu_util.FORMS[request.param]
    yield request.param
    gpu_util.TILE_FORM[0] = gpu_util.FORMS["auto"]
