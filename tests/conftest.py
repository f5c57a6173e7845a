import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
GOLDEN = os.path.join(ROOT, "tests", "golden")
if GOLDEN not in sys.path:
    sys.path.insert(0, GOLDEN)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity and barrier tests")
    config.addinivalue_line("markers", "slow: long CPU-side oracle runs")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_helpers():
    """The oracle and the input generator are plain gcc builds; make sure they exist."""
    import oracle
    from iterative_stencil_pde_amd import inputs
    oracle.build(force=False)
    inputs.build(force=False)
