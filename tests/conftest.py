import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")


def _ensure_host_libs():
    # The CPU-side libraries are plain gcc builds; build them if nothing is built yet.
    import oracle
    import synth
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    if not os.path.exists(synth._LIB_PATH):
        synth.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
