import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the HIP library")


@pytest.fixture(scope="session")
def lowbit_lib():
    """The C-ABI library, built in-tree first if nothing is built yet."""
    from bit_groupwise_weight_amd import lowbit
    if not os.path.exists(lowbit.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return lowbit.load()
