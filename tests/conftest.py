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


def pytest_terminal_summary(terminalreporter):
    """Worst err/tol of the output comparisons of the GPU tests (when any ran):
    the headroom against 1e-3 + 2e-3 * sum |x*w| per case family."""
    helpers = sys.modules.get("tests.gpu_helpers")
    log = getattr(helpers, "ERR_TOL_LOG", None)
    if not log:
        return
    fam = {}
    for what, r in log:
        key = what.split(":")[0].split(" M=")[0]
        if r >= fam.get(key, (-1.0, ""))[0]:
            fam[key] = (r, what)
    terminalreporter.write_sep("-", f"worst err/tol over {len(log)} output comparisons")
    for key, (r, what) in sorted(fam.items(), key=lambda kv: -kv[1][0])[:40]:
        terminalreporter.write_line(f"{r:8.4f}  {what}")
