"""The torch-facing layer without a GPU: op registration, the shape (fake)
functions that torch.compile relies on, argument checks and the
quantize-then-swap flow, all on the meta device."""
import pytest
import torch

from bit_groupwise_weight_amd import nn as lnn

META = torch.device("meta")


def meta_weights(N, K, bits, group, dtype):
    packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=META)
    scales = torch.empty((N, K // group), dtype=dtype, device=META)
    return packed, scales, torch.empty_like(scales)


def test_ops_registered():
    assert hasattr(torch.ops.lowbit, "linear")
    assert hasattr(torch.ops.lowbit, "quantize_pack")
    assert hasattr(torch.ops.lowbit, "linear_a8")


@pytest.mark.parametrize("lead", [(), (5,), (2, 3)])
def test_linear_a8_shape_function(lead):
    N, K, bits, group = 40, 256, 4, 32
    packed, s, z = meta_weights(N, K, bits, group, torch.bfloat16)
    x = torch.empty((*lead, K), dtype=torch.bfloat16, device=META)
    y = torch.ops.lowbit.linear_a8(x, packed, s, z, None, bits, group)
    assert y.shape == (*lead, N) and y.dtype == torch.bfloat16 and y.device == META


def test_module_act_bits():
    m = lnn.LowbitLinear(128, 32, 4, 32, dtype=torch.bfloat16, device=META, act_bits=8)
    assert "act_bits=8" in repr(m)
    y = m(torch.empty((3, 128), dtype=torch.bfloat16, device=META))
    assert y.shape == (3, 32)
    with pytest.raises(ValueError):
        lnn.LowbitLinear(128, 32, 4, 32, act_bits=4)


@pytest.mark.parametrize("bits", range(1, 8))
@pytest.mark.parametrize("lead", [(), (5,), (2, 3)])
def test_linear_shape_function(bits, lead):
    N, K, group = 48, 256, 64
    packed, s, z = meta_weights(N, K, bits, group, torch.float16)
    x = torch.empty((*lead, K), dtype=torch.float16, device=META)
    y = torch.ops.lowbit.linear(x, packed, s, z, None, bits, group)
    assert y.shape == (*lead, N) and y.dtype == torch.float16 and y.device == META


def test_linear_shape_function_fake_mode():
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode():
        packed = torch.empty((24, 128 * 3 // 8), dtype=torch.uint8)
        s = torch.empty((24, 4), dtype=torch.bfloat16)
        x = torch.empty((7, 128), dtype=torch.bfloat16)
        y = torch.ops.lowbit.linear(x, packed, s, s.clone(), torch.empty(24, dtype=torch.bfloat16), 3, 32)
        assert y.shape == (7, 24) and y.dtype == torch.bfloat16


@pytest.mark.parametrize("bad", ["K", "packed", "dtype", "bias", "bits", "group"])
def test_linear_shape_checks(bad):
    N, K, bits, group = 16, 128, 4, 32
    packed, s, z = meta_weights(N, K, bits, group, torch.float16)
    x = torch.empty((2, K), dtype=torch.float16, device=META)
    bias = None
    if bad == "K":
        x = torch.empty((2, K + 32), dtype=torch.float16, device=META)
    elif bad == "packed":
        packed = torch.empty((N, K * bits // 8 - 1), dtype=torch.uint8, device=META)
    elif bad == "dtype":
        x = x.to(torch.bfloat16)
    elif bad == "bias":
        bias = torch.empty((N + 1,), dtype=torch.float16, device=META)
    elif bad == "bits":
        bits = 8
    elif bad == "group":
        group = 48
    with pytest.raises(ValueError):
        torch.ops.lowbit.linear(x, packed, s, z, bias, bits, group)


@pytest.mark.parametrize("bits", [1, 4, 7])
def test_quantize_pack_shape_function(bits):
    w = torch.empty((40, 256), dtype=torch.float32, device=META)
    packed, s, z = torch.ops.lowbit.quantize_pack(w, bits, 128, torch.bfloat16)
    assert packed.shape == (40, 256 * bits // 8) and packed.dtype == torch.uint8
    assert s.shape == z.shape == (40, 2) and s.dtype == z.dtype == torch.bfloat16


def test_module_buffers_and_forward_shape():
    m = lnn.LowbitLinear(256, 80, bits=5, group_size=64, bias=True, dtype=torch.float16, device=META)
    assert m.packed.shape == (80, 160) and m.scales.shape == (80, 4) and m.bias.shape == (80,)
    y = m(torch.empty((3, 4, 256), dtype=torch.float16, device=META))
    assert y.shape == (3, 4, 80)
    assert "bits=5" in repr(m)


def test_module_rejects_bad_config():
    with pytest.raises(ValueError):
        lnn.LowbitLinear(100, 8, bits=4, group_size=64, device=META)
    with pytest.raises(ValueError):
        lnn.LowbitLinear(128, 8, bits=0, group_size=64, device=META)
    with pytest.raises(ValueError):
        lnn.LowbitLinear(128, 8, bits=4, group_size=64, dtype=torch.float64, device=META)


def test_quantize_linears_swaps_on_meta():
    model = torch.nn.Sequential(
        torch.nn.Linear(256, 128, dtype=torch.float16, device=META),
        torch.nn.ReLU(),
        torch.nn.Sequential(torch.nn.Linear(128, 64, bias=False, dtype=torch.float16, device=META),
                            torch.nn.Linear(64, 30, dtype=torch.float16, device=META)),
        torch.nn.Linear(30, 8, dtype=torch.float16, device=META),   # K not a multiple of 64: kept
    )
    lnn.quantize_linears(model, bits=3, group_size=64,
                         filter_fn=lambda mod, name: name != "2.1")
    assert isinstance(model[0], lnn.LowbitLinear) and model[0].bits == 3
    assert isinstance(model[2][0], lnn.LowbitLinear) and model[2][0].bias is None
    assert isinstance(model[2][1], torch.nn.Linear)          # excluded by the filter
    assert isinstance(model[3], torch.nn.Linear)             # 30 % 64 != 0
    y = model[0](torch.empty((2, 256), dtype=torch.float16, device=META))
    assert y.shape == (2, 128)


def test_cpu_tensors_are_rejected():
    """The real op runs only on the GPU: CPU inputs raise instead of computing."""
    packed = torch.zeros((8, 64), dtype=torch.uint8)
    s = torch.zeros((8, 4), dtype=torch.float16)
    x = torch.zeros((1, 128), dtype=torch.float16)
    with pytest.raises((ValueError, RuntimeError)):
        torch.ops.lowbit.linear(x, packed, s, s.clone(), None, 4, 32)
