import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size shapes (minutes of CPU)")


@pytest.fixture(scope="session", autouse=True)
def _synth_built():
    # the seeded input generator is a small gcc build; compile it if absent
    import synth

    if not os.path.exists(synth._LIB_PATH):
        synth.build()
    yield
