"""The measurement instruments of the library (not part of the layer): the
pointer chase ends where following the chain on the host ends, with links
out of range clamped to the last element; the streaming read returns without
error and leaves the sink alone unless the data fold to its constant."""
import numpy as np
import pytest
import torch

from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd import probe
from tests.gpu_helpers import DEV

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(autouse=True)
def _lib(lowbit_lib):
    yield


def host_chase(chain, hops, start):
    i, last = start, len(chain) - 1
    for _ in range(hops):
        i = min(int(chain[i]), last)
    return i


@pytest.mark.parametrize("hops", [0, 1, 7, 1000])
def test_chase_matches_host(hops):
    rng = np.random.default_rng(hops)
    n = 4099
    chain = rng.integers(0, n, size=n, dtype=np.int64).astype(np.uint32)
    chain[::17] = np.uint32(0xFFFFFFF0)          # out-of-range links are clamped
    out = torch.zeros(1, dtype=torch.int32, device=DEV)
    probe.chase(torch.from_numpy(chain.view(np.int32)).to(DEV), hops, 5, out)
    torch.cuda.synchronize()
    assert int(out.item()) == host_chase(chain, hops, 5)


@pytest.mark.parametrize("lpt", [1, 2, 4, 8])
@pytest.mark.parametrize("nbytes", [16, 4096, 3 * 4096 + 48, 9453568])
def test_stream_read_runs(nbytes, lpt):
    src = torch.zeros(nbytes + 256, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    probe.stream_read(src, nbytes, lpt, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7       # zeros fold to 0, not the constant
