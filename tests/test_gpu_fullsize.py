"""Full-size workloads compared over EVERY output element and every code,
scale and zero, in the launch configuration the benchmark times (default
dispatch, default workspace):

  * batched (MFMA): M=128, bits 4, group 128, bf16, (K, N) = (4096, 14336)
    and (14336, 4096) -- every column tile and K split of the production
    schedule;
  * Llama-3.1-8B decode: M=1, group 64, fp16, (K, N) = (4096, 14336) and
    (14336, 4096) at bits 1, 4 and 7;
  * mixed sweep at M=64: K=N=4096, fp16 with bias, bits 1, 2, 4, 7 and every
    group size.

GPU quantize -> GPU linear; the oracle quantizes the whole weight and
computes the whole output in fp64.  (Every workload configuration is also
covered, on sampled rows, by tests/test_gpu_parity.py.)
"""
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd.workloads import batched_qmm, llama8b_decode, make_bias, make_x, mixed_sweep
from tests.gpu_helpers import DEV, TORCH_ACT, bias_values, check_close, weight_for, x_values
from tests.test_gpu_parity import assert_quant_equal

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module", autouse=True)
def _lib(lowbit_lib):
    return lowbit_lib


FULL_CASES = (batched_qmm()
              + [c for c in llama8b_decode() if (c.K, c.N) in ((4096, 14336), (14336, 4096))
                 and c.bits in (1, 4, 7)]
              + [c for c in mixed_sweep() if c.M == 64])


@pytest.mark.parametrize("case", FULL_CASES, ids=[c.name for c in FULL_CASES])
def test_workload_full_output(case):
    print(f"full-size {case.name}: M={case.M} K={case.K} N={case.N} b={case.bits} g={case.group} "
          f"{case.act}", flush=True)
    W = weight_for(case)
    x = make_x(case)
    b = make_bias(case)
    packed, s, z, codes = lb.lowbit_quantize_pack(W.to(DEV), case.bits, case.group, TORCH_ACT[case.act],
                                                  want_codes=True)
    y = lb.lowbit_linear(x.to(DEV), packed, s, z, None if b is None else b.to(DEV), case.bits, case.group)
    torch.cuda.synchronize()
    ref = oracle.quantize(W.numpy(), case.bits, case.group, case.act)
    assert_quant_equal(ref, packed, s, z, codes, case.bits)
    y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], case.group, bias_values(b))
    assert y.shape == y_ref.shape
    check_close(y, y_ref, A, f"full {case.name}")
