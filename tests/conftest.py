import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _name_parity_records(request):
    """Parity comparisons made during a test are recorded under its id (when
    RA_PARITY_LOG names a file; see tests/helpers.py)."""
    from tests import helpers
    helpers.CURRENT_TEST = request.node.nodeid
    yield
    helpers.CURRENT_TEST = None
