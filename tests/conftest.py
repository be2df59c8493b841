import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    """gen/ and oracle/ are plain C: build them once if they are missing."""
    import gen
    import oracle.moe
    gen.build(force=False)
    oracle.moe.build(force=False)
    yield
