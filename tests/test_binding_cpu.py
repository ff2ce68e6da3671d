"""Argument checks of the Python binding (no GPU needed).

The C interface takes raw pointers and cannot see buffer sizes or dtypes, so
the binding checks every tensor's shape, dtype and device before it hands a
pointer over: a buffer smaller than the kernels assume must be refused here,
not read past on the GPU.  With CPU tensors every correctly shaped call ends
at the device check, so each case below shows which check fires first.
"""
import pytest
import torch

from bit_groupwise_weight_amd import lowbit as lb


@pytest.fixture(scope="module", autouse=True)
def _lib(lowbit_lib):
    return lowbit_lib


N, K, BITS, GROUP = 8, 128, 4, 32


def weights(dtype=torch.float16, bits=BITS):
    packed = torch.zeros(N * K * bits // 8, dtype=torch.uint8)
    scales = torch.zeros(N, K // GROUP, dtype=dtype)
    return packed, scales, scales.clone()


def linear(x, packed, scales, zeros, bias=None, y=None, bits=BITS, group=GROUP):
    return lb.lowbit_linear(x, packed, scales, zeros, bias, bits, group, y=y)


def test_linear_reaches_device_check_when_shapes_are_right():
    x = torch.zeros(2, K, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU memory"):
        linear(x, *weights())


@pytest.mark.parametrize("case, match", [
    ("packed_short", "packed holds"),
    ("packed_dtype", "packed must be uint8"),
    ("scales_shape", "scales must be"),
    ("zeros_dtype", "zeros must be"),
    ("bias_shape", "bias must be"),
    ("y_shape", "y must be"),
    ("x_dtype", "x dtype"),
    ("x_1d", "x must be 2-D"),
    ("bits", "bits must be"),
    ("group", "group must be"),
])
def test_linear_refuses_bad_tensors(case, match):
    x = torch.zeros(2, K, dtype=torch.float16)
    packed, scales, zeros = weights()
    bias = y = None
    bits, group = BITS, GROUP
    if case == "packed_short":
        packed = packed[:-1]
    elif case == "packed_dtype":
        packed = packed.to(torch.int8)
    elif case == "scales_shape":
        scales = torch.zeros(N, K // GROUP + 1, dtype=torch.float16)
    elif case == "zeros_dtype":
        zeros = zeros.to(torch.bfloat16)
    elif case == "bias_shape":
        bias = torch.zeros(N + 1, dtype=torch.float16)
    elif case == "y_shape":
        y = torch.zeros(2, N + 1, dtype=torch.float16)
    elif case == "x_dtype":
        x = x.to(torch.float64)
    elif case == "x_1d":
        x = x[0]
    elif case == "bits":
        bits = 8
    elif case == "group":
        group = 48
    with pytest.raises(ValueError, match=match):
        linear(x, packed, scales, zeros, bias, y, bits, group)


def test_multi_refuses_mismatched_rows_and_short_weights():
    x = torch.zeros(2, K, dtype=torch.float16)
    packed, scales, zeros = weights()
    with pytest.raises(ValueError, match="same M"):
        lb.lowbit_linear_multi([(x, packed, scales, zeros, None, None),
                                (x[:1], packed, scales, zeros, None, None)], BITS, GROUP)
    with pytest.raises(ValueError, match="packed holds"):
        lb.lowbit_linear_multi([(x, packed, scales, zeros, None, None),
                                (x, packed[:10], scales, zeros, None, None)], BITS, GROUP)


def test_quantize_refuses_bad_outputs_and_input():
    w = torch.zeros(N, K)
    packed, scales, zeros = weights()
    with pytest.raises(ValueError, match="packed holds"):
        lb.lowbit_quantize_pack(w, BITS, GROUP, torch.float16, out=(packed[:-3], scales, zeros, None))
    with pytest.raises(ValueError, match="scales must be"):
        lb.lowbit_quantize_pack(w, BITS, GROUP, torch.float16, out=(packed, scales[:, :1], zeros, None))
    with pytest.raises(ValueError, match="codes must be"):
        lb.lowbit_quantize_pack(w, BITS, GROUP, torch.float16,
                                out=(packed, scales, zeros, torch.zeros(N, K - 1, dtype=torch.uint8)))
    with pytest.raises(ValueError, match="w must be float32, float16 or bfloat16"):
        lb.lowbit_quantize_pack(w.double(), BITS, GROUP, torch.float16)
    with pytest.raises(ValueError, match="GPU memory"):
        lb.lowbit_quantize_pack(w, BITS, GROUP, torch.float16, out=(packed, scales, zeros, None))


def test_prepared_linear_checks_weights_once_at_construction():
    packed, scales, zeros = weights()
    with pytest.raises(ValueError, match="packed holds"):
        lb.PreparedLinear(packed[:-1], scales, zeros, None, BITS, GROUP)
    with pytest.raises(ValueError, match="bias must be"):
        lb.PreparedLinear(packed, scales, zeros, torch.zeros(N + 1, dtype=torch.float16), BITS, GROUP)
    with pytest.raises(ValueError, match="zeros must be"):
        lb.PreparedLinear(packed, scales, zeros.to(torch.bfloat16), None, BITS, GROUP)
    with pytest.raises(ValueError, match="GPU memory"):
        lb.PreparedLinear(packed, scales, zeros, None, BITS, GROUP)


@pytest.mark.parametrize("case", [
    dict(bits=8), dict(group=48), dict(M=0), dict(M=-1), dict(x=0), dict(x=0x10004),
    dict(packed=0x10008), dict(ws=0, ws_bytes=64), dict(act=7), dict(N=0), dict(K=96),
    dict(bias=0x10000, M=0)])
def test_fastcall_passes_arguments_unchanged(case):
    """The compiled marshalling module of PreparedLinear hands lowbit_linear
    the same arguments as ctypes: on calls the library settles before any
    HIP call (argument errors, M = 0), status and message agree."""
    import ctypes
    fc = lb._fastcall_module()
    if fc is None:
        pytest.skip("the marshalling module is not built")
    lib = lb.load()
    a = dict(x=0x10000, act=1, packed=0x10000, scales=0x10000, zeros=0x10000, bias=None,
             y=0x10000, bits=4, group=64, M=1, N=64, K=256, ws=0, ws_bytes=0)
    a.update(case)
    vp = lambda v: ctypes.c_void_p(v or None)
    st_ct = lib.lowbit_linear(vp(a["x"]), a["act"], vp(a["packed"]), vp(a["scales"]),
                              vp(a["zeros"]), vp(a["bias"]), vp(a["y"]), a["bits"], a["group"],
                              ctypes.c_int64(a["M"]), ctypes.c_int64(a["N"]), ctypes.c_int64(a["K"]),
                              vp(a["ws"]), ctypes.c_size_t(a["ws_bytes"]), None)
    msg_ct = lb.lowbit_last_error()
    fn = ctypes.cast(lib.lowbit_linear, ctypes.c_void_p).value
    bound = fc.bind(fn, a["act"], a["packed"], a["scales"], a["zeros"], a["bias"], a["bits"],
                    a["group"], a["N"], a["K"])
    st_fc = fc.call(bound, a["x"], a["y"], a["M"], a["ws"], a["ws_bytes"], 0)
    assert st_fc == st_ct
    if st_ct != 0:
        assert lb.lowbit_last_error() == msg_ct


def test_fastcall_rejects_bad_arity():
    fc = lb._fastcall_module()
    if fc is None:
        pytest.skip("the marshalling module is not built")
    with pytest.raises(TypeError):
        fc.call(1, 2)
    with pytest.raises(TypeError):
        fc.bind(1)
