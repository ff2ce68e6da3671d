"""lowbit_linear_multi: several decode linears in one launch give exactly the
results of separate decode-path calls, and match the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd.workloads import Case, make_weight, make_x
from tests.gpu_helpers import DEV, TORCH_ACT, check_close, upload_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(lowbit_lib):
    yield


def quantized(N, K, bits, group, act, seed):
    case = Case("m", 1, K, N, bits, group, act, seed=seed)
    ref = oracle.quantize(make_weight(case).numpy(), bits, group, act)
    return ref, upload_quant(ref["q"], ref["s"], ref["z"], bits, act)


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bits", [1, 3, 4, 7])
@pytest.mark.parametrize("M", [1, 3])
def test_multi_equals_separate_calls_and_oracle(bits, act, M):
    group = 64
    # q/k/v-like (shared x, different N), plus one with another K and its own x and a bias
    shapes = [(200, 512), (64, 512), (64, 512), (96, 1536)]
    xs = {K: make_x(Case("x", M, K, 1, bits, group, act, seed=K + M)) for _, K in set(shapes)}
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        ref, (packed, s, z) = quantized(N, K, bits, group, act, seed=10 * i + bits)
        b = (torch.randn(N, generator=torch.Generator().manual_seed(i)) * 0.1).to(TORCH_ACT[act]) \
            if i == 3 else None
        items.append((xs[K].to(DEV), packed, s, z, None if b is None else b.to(DEV), None))
        refs.append((ref, b, K))
    outs = lb.lowbit_linear_multi(items, bits, group)
    torch.cuda.synchronize()
    for (x, packed, s, z, b, _), y, (ref, bref, K) in zip(items, outs, refs):
        single = lb.lowbit_linear(x, packed, s, z, b, bits, group, path=lb.PATH_QMV)
        torch.cuda.synchronize()
        assert torch.equal(y, single)
        y_ref, A = oracle.linear(x.float().cpu().numpy(), ref["q"], ref["s"], ref["z"], group,
                                 None if bref is None else bref.float().numpy())
        check_close(y, y_ref, A, f"multi b={bits} {act} M={M} K={K}")


def test_multi_llama_layer_shapes():
    """Llama-3.1-8B decode shapes at b=4, g=64: q/k/v in one launch, gate/up in one."""
    bits, group, act = 4, 64, "f16"
    x = make_x(Case("x", 1, 4096, 1, bits, group, act, seed=5)).to(DEV)
    for shapes in ([(4096, 4096), (1024, 4096), (1024, 4096)], [(14336, 4096), (14336, 4096)]):
        items = []
        for i, (N, K) in enumerate(shapes):
            W = torch.randn((N, K), generator=torch.Generator().manual_seed(i)) * 0.02
            packed, s, z, _ = lb.lowbit_quantize_pack(W.to(DEV), bits, group, torch.float16)
            items.append((x, packed, s, z, None, None))
        outs = lb.lowbit_linear_multi(items, bits, group)
        for (xx, packed, s, z, _, _), y in zip(items, outs):
            assert torch.equal(y, lb.lowbit_linear(xx, packed, s, z, None, bits, group, path=lb.PATH_QMV))


@pytest.mark.parametrize("chunk", range(12))
def test_multi_random_mixes(chunk):
    """Seeded random mixes of 1-8 problems in one launch: every N from 1 to
    1200, K from one group to 12288 (one to three rounds per lane, lane
    groups of different widths side by side), M from 1 to 6, with and
    without bias; each output equals its separate decode-path call bit for
    bit and matches the oracle."""
    rng = np.random.default_rng(0xA11 + chunk)
    bits = int(rng.integers(1, 8))
    group = [32, 64, 128, 256][int(rng.integers(4))]
    act = ["f32", "f16", "bf16"][int(rng.integers(3))]
    M = int(rng.integers(1, 7))
    count = int(rng.integers(1, lb.MAX_MULTI + 1))
    items, refs = [], []
    for i in range(count):
        N = int(rng.integers(1, 1201))
        K = group * int(rng.integers(1, 12288 // group + 1))
        ref, (packed, s, z) = quantized(N, K, bits, group, act, seed=100 * chunk + i)
        x = make_x(Case("x", M, K, 1, bits, group, act, seed=1000 * chunk + i))
        b = None
        if rng.integers(2):
            b = (torch.randn(N, generator=torch.Generator().manual_seed(i)) * 0.1).to(TORCH_ACT[act])
        items.append((x.to(DEV), packed, s, z, None if b is None else b.to(DEV), None))
        refs.append((ref, x, b, N, K))
    outs = lb.lowbit_linear_multi(items, bits, group)
    torch.cuda.synchronize()
    for (xd, packed, s, z, bd, _), y, (ref, x, b, N, K) in zip(items, outs, refs):
        what = f"multi chunk={chunk} b={bits} g={group} {act} M={M} N={N} K={K}"
        single = lb.lowbit_linear(xd, packed, s, z, bd, bits, group, path=lb.PATH_QMV)
        torch.cuda.synchronize()
        assert torch.equal(y, single), what
        y_ref, A = oracle.linear(x.float().numpy(), ref["q"], ref["s"], ref["z"], group,
                                 None if b is None else b.float().numpy())
        check_close(y, y_ref, A, what)
