import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def mk():
    """The product binding; builds libmla_kv.so first if it is missing."""
    import fp8_paged_insert_amd as mk_
    from fp8_paged_insert_amd import build as hipbuild

    if not os.path.exists(mk_.LIB_PATH):
        hipbuild.build()
    mk_.lib()
    return mk_
