import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import pao
    return pao.load_library()


def pytest_terminal_summary(terminalreporter):
    """The worst error of every oracle comparison a test asked to report:
    fp32 max abs error (bound 1e-5), bf16 worst per-row relative error
    (bound 1e-2)."""
    from tests import helpers
    if not helpers.MARGINS:
        return
    tr = terminalreporter
    tr.section("error margins against the float64 oracle")
    for what, dtype, rows, err, bound in helpers.MARGINS:
        kind = "max abs err" if dtype == "f32" else "worst row rel err"
        tr.write_line(f"{what}: {rows} rows, {kind} {err:.3e} (bound {bound:.0e}, "
                      f"{err / bound:.3f} of it)")
