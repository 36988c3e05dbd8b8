import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running parity case")


def _ensure_host_libs():
    """Build the oracle and the host generator if they are missing (gcc only,
    a second or two).  The HIP library is built by __graft_entry__.build()."""
    need = [os.path.join(ROOT, "oracle", "libmoe_oracle.so"),
            os.path.join(ROOT, "gen", "libmoe_gen.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build_host()


_ensure_host_libs()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
