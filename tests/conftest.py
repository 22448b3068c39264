import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionfinish(session, exitstatus):
    """The 1e-5 tie-mismatch rate over every code the session compared
    (tests/parity.py keeps the tally).  A session that compared fewer than a
    million codes cannot resolve the rate and says so; otherwise a rate above
    1e-5 fails the session."""
    try:
        from tests.parity import TALLY
    except Exception:
        return
    n, m = TALLY["elements"], TALLY["mismatch"]
    if n == 0:
        return
    rate = m / n
    tr = session.config.pluginmanager.get_plugin("terminalreporter")
    msg = f"code tie mismatches over the session: {m} of {n} compared codes (rate {rate:.2e})"
    if n < 1_000_000:
        msg += "; too few codes to resolve a 1e-5 rate"
    elif rate > 1e-5:
        msg += " exceeds 1e-5"
        session.exitstatus = pytest.ExitCode.TESTS_FAILED
    if tr is not None:
        tr.write_line(msg)
