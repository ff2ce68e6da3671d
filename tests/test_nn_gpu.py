"""The torch-facing layer on the GPU: LowbitLinear against the CPU oracle,
torch.compile through the registered ops, and the quantize-then-swap flow."""
import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import nn as lnn
from bit_groupwise_weight_amd.workloads import Case, make_weight, make_x
from tests.gpu_helpers import DEV, TORCH_ACT, check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(lowbit_lib):
    yield


def module_case(bits, group, act, bias, seed, N=96, K=512):
    case = Case("nn", 1, K, N, bits, group, act, bias=bias, seed=seed)
    W = make_weight(case)                       # fp32 [N, K]
    b = (torch.randn(N, generator=torch.Generator().manual_seed(seed + 2)) * 0.1).to(TORCH_ACT[act]) \
        if bias else None
    return case, W, b


def oracle_forward(W, b, x2, bits, group, act):
    ref = oracle.quantize(W.numpy(), bits, group, act)
    y, A = oracle.linear(x2.float().numpy(), ref["q"], ref["s"], ref["z"], group,
                         None if b is None else b.float().numpy())
    return y, A


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_module_matches_oracle(bits, act):
    group = [32, 64, 128, 256][bits % 4]
    case, W, b = module_case(bits, group, act, bias=bits % 2 == 1, seed=100 + bits)
    lin = torch.nn.Linear(case.K, case.N, bias=b is not None, device=DEV, dtype=torch.float32)
    with torch.no_grad():
        lin.weight.copy_(W.to(DEV))
        if b is not None:
            lin.bias.copy_(b.float().to(DEV))
    m = lnn.LowbitLinear.from_linear(lin, bits, group, dtype=TORCH_ACT[act])
    x = torch.randn((2, 3, case.K), generator=torch.Generator().manual_seed(bits)).to(TORCH_ACT[act])
    y = m(x.to(DEV))
    assert y.shape == (2, 3, case.N) and y.dtype == TORCH_ACT[act]
    y_ref, A = oracle_forward(W, b, x.reshape(-1, case.K), bits, group, act)
    check_close(y.reshape(-1, case.N), y_ref, A, f"LowbitLinear b={bits} g={group} {act}")
    # the module's quantized state is the oracle's, bit for bit
    ref = oracle.quantize(W.numpy(), bits, group, act)
    assert np.array_equal(m.packed.cpu().numpy(), oracle.pack(ref["q"], bits))


def test_compile_matches_eager():
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(256, 512), torch.nn.GELU(), torch.nn.Linear(512, 128))
    model = model.to(DEV).to(torch.bfloat16)
    lnn.quantize_linears(model, bits=4, group_size=128)
    x = torch.randn((4, 256), device=DEV, dtype=torch.bfloat16)
    eager = model(x)
    compiled = torch.compile(model, fullgraph=True, backend="aot_eager")
    out = compiled(x)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)


def test_quantize_linears_mlp_matches_oracle():
    torch.manual_seed(1)
    l1, l2 = torch.nn.Linear(384, 256), torch.nn.Linear(256, 64, bias=False)
    model = torch.nn.Sequential(l1, torch.nn.ReLU(), l2).to(DEV).to(torch.float16)
    W1, b1, W2 = l1.weight.detach().float().cpu(), l1.bias.detach().cpu(), l2.weight.detach().float().cpu()
    lnn.quantize_linears(model, bits=6, group_size=64)
    assert isinstance(model[0], lnn.LowbitLinear) and isinstance(model[2], lnn.LowbitLinear)
    x = torch.randn((5, 384), dtype=torch.float16)
    h = model[0](x.to(DEV))
    h_ref, A = oracle_forward(W1, b1, x, 6, 64, "f16")
    check_close(h, h_ref, A, "layer 1")
    y = model[2](torch.relu(h))
    y_ref, A2 = oracle_forward(W2, None, torch.relu(h).cpu(), 6, 64, "f16")
    check_close(y, y_ref, A2, "layer 2")


@pytest.mark.parametrize("M,act,bits,group,bias", [
    (1, "f16", 4, 64, True), (3, "bf16", 7, 32, False), (1, "f32", 2, 128, True),
    (40, "bf16", 4, 128, True), (96, "f16", 3, 256, False)])
def test_prepared_call_matches_lowbit_linear(M, act, bits, group, bias):
    """The prepared eager call is lowbit_linear with the weights bound once:
    the same output bit for bit (decode and MFMA paths, with and without a K
    split), with a preallocated y and an explicit stream too."""
    from bit_groupwise_weight_amd import lowbit as lb
    case, W, b = module_case(bits, group, act, bias, seed=M + bits, N=200, K=1024)
    dt = TORCH_ACT[act]
    packed, s, z = lnn.quantize_pack(W.to(DEV), bits, group, dt)
    bd = None if b is None else b.to(DEV)
    x = torch.randn((M, case.K), generator=torch.Generator().manual_seed(M)).to(dt).to(DEV)
    y_ref = lb.lowbit_linear(x, packed, s, z, bd, bits, group)
    call = lb.PreparedLinear(packed, s, z, bd, bits, group)
    y1 = call(x)
    y2 = torch.full_like(y_ref, float("nan"))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    call(x, y=y2, stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(y1, y_ref) and torch.equal(y2, y_ref)
    with pytest.raises(ValueError, match="x must be"):
        call(x[:, :-32].contiguous())


def test_module_rebinds_replaced_buffers():
    """Buffers replaced after the first call (as .to() or assignment does) are
    the ones the next eager call reads."""
    case, W, b = module_case(4, 64, "f16", True, seed=9, N=64, K=256)
    m = lnn.LowbitLinear(case.K, case.N, 4, 64, bias=True, dtype=torch.float16, device=DEV)
    m.set_weight(W.to(DEV), b.to(DEV))
    x = torch.randn((2, case.K), generator=torch.Generator().manual_seed(3)).half().to(DEV)
    y0 = m(x)
    m.scales = m.scales.clone()
    m.zeros = torch.zeros_like(m.zeros)
    y1 = m(x)
    op = torch.ops.lowbit.linear(x, m.packed, m.scales, m.zeros, m.bias, 4, 64)
    torch.cuda.synchronize()
    assert torch.equal(y1, op) and not torch.equal(y0, y1)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_module_act_bits_matches_oracle(act):
    # 8-bit dynamic activations: the oracle's int8 codes of x, then its linear
    bits, group = 4, 32
    case, W, b = module_case(bits, group, act, bias=True, seed=7, N=130, K=416)
    lin = torch.nn.Linear(case.K, case.N, device=DEV, dtype=torch.float32)
    with torch.no_grad():
        lin.weight.copy_(W.to(DEV))
        lin.bias.copy_(b.float().to(DEV))
    m = lnn.LowbitLinear.from_linear(lin, bits, group, dtype=TORCH_ACT[act], act_bits=8)
    x = torch.randn((2, 5, case.K), generator=torch.Generator().manual_seed(3)).to(TORCH_ACT[act])
    y = m(x.to(DEV))
    assert y.shape == (2, 5, case.N) and y.dtype == TORCH_ACT[act]
    ref = oracle.quantize(W.numpy(), bits, group, act)
    xq, a = oracle.quantize_activations_i8(x.reshape(-1, case.K).float().numpy())
    y_ref, A = oracle.linear_a8(xq, a, ref["q"], ref["s"], ref["z"], group, b.float().numpy())
    check_close(y.reshape(-1, case.N), y_ref, A, f"LowbitLinear act_bits=8 {act}")


def test_act_bits_compile_matches_eager():
    torch.manual_seed(1)
    model = torch.nn.Sequential(torch.nn.Linear(256, 512), torch.nn.GELU(), torch.nn.Linear(512, 128))
    model = model.to(DEV).to(torch.bfloat16)
    lnn.quantize_linears(model, bits=4, group_size=32, act_bits=8)
    x = torch.randn((20, 256), device=DEV, dtype=torch.bfloat16)
    eager = model(x)
    compiled = torch.compile(model, fullgraph=True, backend="aot_eager")
    out = compiled(x)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
