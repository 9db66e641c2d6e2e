import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def ref():
    """The normal CPU oracle build (compiled on first use if missing)."""
    import oracle
    return oracle.load()


@pytest.fixture(scope="session")
def mutant(tmp_path_factory):
    """Build a deliberately wrong variant of the oracle (teeth for the pins)."""
    import oracle
    cache = {}

    def get(define: str):
        if define not in cache:
            path = str(tmp_path_factory.mktemp("mutant") / f"lib_{define}.so")
            oracle.build(path, defines=(define,))
            cache[define] = oracle.Oracle(path)
        return cache[define]

    return get
