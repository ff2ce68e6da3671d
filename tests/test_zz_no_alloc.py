"""lowbit_linear_noalloc (the entry point that allocates nothing) against
lowbit_linear with a full workspace -- the same schedule and kernels, so the
outputs must be bitwise equal -- and against the oracle's tolerance, on two
calls in a row, the second with a smaller problem (the library's device array
keeps the first call's partial planes; the second must not depend on them)."""
import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd.workloads import Case, make_bias, make_x
from tests.gpu_helpers import DEV, TORCH_ACT, check_close, upload_quant, weight_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module", autouse=True)
def _lib(lowbit_lib):
    return lowbit_lib


def _prepare(case):
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, case.bits, case.group, case.act)
    x, b = make_x(case), make_bias(case)
    y_ref, A = oracle.linear(x.float().numpy(), ref["q"], ref["s"], ref["z"], case.group,
                             None if b is None else b.float().numpy())
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], case.bits, case.act)
    xd, bd = x.to(DEV), None if b is None else b.to(DEV)
    return xd, packed, s, z, bd, y_ref, A


# (larger first, then smaller): MFMA schedules with K splits of different
# plane counts and sizes, then a decode-kernel case that uses no scratch
SEQUENCES = [
    [Case("na0", 128, 4096, 4096, 4, 128, "bf16", bias=True, seed=3),
     Case("na1", 40, 1024, 520, 3, 64, "f16", bias=False, seed=4)],
    [Case("na2", 96, 2048, 3000, 5, 32, "f16", bias=True, seed=5),
     Case("na3", 17, 512, 130, 2, 256, "bf16", bias=True, seed=6),
     Case("na4", 3, 1024, 200, 7, 32, "f16", bias=True, seed=7)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_call(seq):
    for case in SEQUENCES[seq]:
        xd, packed, s, z, bd, y_ref, A = _prepare(case)
        M, N, K = case.M, case.N, case.K
        need = lb.lowbit_linear_workspace_bytes(case.bits, case.group, M, N, K, TORCH_ACT[case.act])
        ws = torch.full((max(need, 1),), 0x5A, dtype=torch.uint8, device=DEV)
        y_ws = lb.lowbit_linear(xd, packed, s, z, bd, case.bits, case.group, workspace=ws)
        y = torch.full((M, N), float("nan"), dtype=TORCH_ACT[case.act], device=DEV)
        lb.lowbit_linear_noalloc(xd, packed, s, z, bd, case.bits, case.group, y=y)
        torch.cuda.synchronize()
        what = f"noalloc {case.name}: M={M} N={N} K={K} b={case.bits} g={case.group} {case.act}"
        assert torch.equal(y, y_ws), what + " differs from lowbit_linear with a workspace"
        check_close(y, y_ref, A, what)


def test_noalloc_requires_y():
    case = SEQUENCES[0][1]
    xd, packed, s, z, bd, _, _ = _prepare(case)
    with pytest.raises(ValueError):
        lb.lowbit_linear_noalloc(xd, packed, s, z, bd, case.bits, case.group, y=None)
