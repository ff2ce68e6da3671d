"""torch-facing layer on top of the C ABI: custom ops and a drop-in linear module.

The issue "Revamp int4 MPS support in torchao" (issue text) asks for a
module built directly on the weight-only quantized linear that quantizes on
the fly and accepts a bias, and its thread shows a user broken by one missing
bit width: here an ``nn.Linear`` is replaced by a module that quantizes its
weight once, keeps the packed codes and the per-group scales and zeros, and
runs the low-bit kernel in ``forward``, for every bit width 1..7.  "Add
support for fbgemm int4 mm kernel" notes that an op without a shape (meta)
function cannot be traced by ``torch.compile``; the ops registered here carry
one.

Ops (namespace ``lowbit``):

* ``lowbit::quantize_pack(Tensor w, int bits, int group, ScalarType sz_dtype)
  -> (Tensor packed, Tensor scales, Tensor zeros)`` -- fp32 ``w[N, K]`` on the
  GPU to codes packed LSB-first, ``N x (K*bits/8)`` bytes, and scales / zeros
  ``N x (K/group)`` in ``sz_dtype``;
* ``lowbit::linear(Tensor x, Tensor packed, Tensor scales, Tensor zeros,
  Tensor? bias, int bits, int group) -> Tensor`` -- ``x[..., K]`` to
  ``y[..., N]`` in x's dtype, ``y = x . dequant(W)^T (+ bias)``;
* ``lowbit::linear_a8(...)`` -- the same signature with 8-bit dynamic
  activations: each row of x is quantized on the fly to int8 codes with one
  fp32 scale (symmetric, max |x| / 127), and the linear runs over the codes
  on the int8 matrix cores (the export mode with 8-bit dynamic activations
  and 4-bit weights in groups of 32 of "[MPS] Add support for Int4 groupwise
  quantization").

Both run in liblowbit.so through :mod:`bit_groupwise_weight_amd.lowbit`;
nothing here computes on the CPU.
"""
from __future__ import annotations

from typing import Callable, Optional, Tuple

import torch

from . import lowbit as _lb

_SZ_DTYPES = (torch.float16, torch.bfloat16, torch.float32)


def _check_bits_group(bits: int, group: int) -> None:
    if bits not in range(1, 8):
        raise ValueError(f"bits must be in 1..7, got {bits}")
    if group not in (32, 64, 128, 256):
        raise ValueError(f"group must be 32, 64, 128 or 256, got {group}")


def _check_linear_shapes(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                         zeros: torch.Tensor, bias: Optional[torch.Tensor], bits: int,
                         group: int) -> Tuple[int, int]:
    _check_bits_group(bits, group)
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension (..., K)")
    K = x.shape[-1]
    if scales.dim() != 2 or zeros.shape != scales.shape:
        raise ValueError("scales and zeros must both be [N, K/group]")
    N = scales.shape[0]
    if K % group != 0 or scales.shape[1] != K // group:
        raise ValueError(f"x has K={K}, scales imply K={scales.shape[1] * group}")
    if packed.numel() != N * K * bits // 8:
        raise ValueError(f"packed holds {packed.numel()} bytes, expected N*K*bits/8 = {N * K * bits // 8}")
    if packed.dtype != torch.uint8:
        raise ValueError("packed must be uint8")
    if scales.dtype != x.dtype or zeros.dtype != x.dtype:
        raise ValueError("scales and zeros must have the activation dtype")
    if bias is not None and (bias.shape != (N,) or bias.dtype != x.dtype):
        raise ValueError("bias must be [N] in the activation dtype")
    return N, K


# ------------------------------------------------------------------ ops --

@torch.library.custom_op("lowbit::quantize_pack", mutates_args=())
def quantize_pack(w: torch.Tensor, bits: int, group: int,
                  sz_dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    _check_bits_group(bits, group)
    if sz_dtype not in _SZ_DTYPES:
        raise ValueError(f"sz_dtype must be one of {_SZ_DTYPES}")
    # fp32, fp16 and bf16 weights go in as they are (the kernel takes fp16 and
    # bf16 values exactly as fp32); other dtypes are converted to fp32 first
    if w.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        w = w.float()
    packed, scales, zeros, _ = _lb.lowbit_quantize_pack(w.contiguous(), bits, group, sz_dtype)
    return packed, scales, zeros


@quantize_pack.register_fake
def _quantize_pack_fake(w, bits, group, sz_dtype):
    _check_bits_group(bits, group)
    N, K = w.shape
    if K % group != 0:
        raise ValueError(f"K={K} is not a multiple of group={group}")
    packed = w.new_empty((N, K * bits // 8), dtype=torch.uint8)
    scales = w.new_empty((N, K // group), dtype=sz_dtype)
    return packed, scales, torch.empty_like(scales)


@torch.library.custom_op("lowbit::linear", mutates_args=())
def linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
           bias: Optional[torch.Tensor], bits: int, group: int) -> torch.Tensor:
    N, K = _check_linear_shapes(x, packed, scales, zeros, bias, bits, group)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K).contiguous()
    y = _lb.lowbit_linear(x2, packed.contiguous(), scales.contiguous(), zeros.contiguous(),
                          None if bias is None else bias.contiguous(), bits, group)
    return y.reshape(*lead, N)


@linear.register_fake
def _linear_fake(x, packed, scales, zeros, bias, bits, group):
    N, _ = _check_linear_shapes(x, packed, scales, zeros, bias, bits, group)
    return x.new_empty((*x.shape[:-1], N))


@torch.library.custom_op("lowbit::linear_a8", mutates_args=())
def linear_a8(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
              bias: Optional[torch.Tensor], bits: int, group: int) -> torch.Tensor:
    N, K = _check_linear_shapes(x, packed, scales, zeros, bias, bits, group)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K).contiguous()
    xq, ascale = _lb.lowbit_quantize_act_i8(x2)
    y = _lb.lowbit_linear_a8(xq, ascale, packed.contiguous(), scales.contiguous(),
                             zeros.contiguous(), None if bias is None else bias.contiguous(),
                             bits, group)
    return y.reshape(*lead, N)


@linear_a8.register_fake
def _linear_a8_fake(x, packed, scales, zeros, bias, bits, group):
    N, _ = _check_linear_shapes(x, packed, scales, zeros, bias, bits, group)
    return x.new_empty((*x.shape[:-1], N))


# --------------------------------------------------------------- module --

class LowbitLinear(torch.nn.Module):
    """``nn.Linear`` with a groupwise b-bit weight: w = s * q + z per group.

    Buffers: ``packed`` (uint8, ``[N, K*bits/8]``), ``scales`` and ``zeros``
    (``[N, K/group]``, activation dtype) and optional ``bias`` (``[N]``).
    Inputs must be on the GPU, in the activation dtype, with last dim K.
    ``act_bits=8`` quantizes the activations too, per row to int8 on every
    call (``lowbit::linear_a8``); ``None`` keeps them floating point.
    """

    def __init__(self, in_features: int, out_features: int, bits: int, group_size: int,
                 bias: bool = True, dtype: torch.dtype = torch.float16,
                 device: Optional[torch.device] = None, act_bits: Optional[int] = None):
        super().__init__()
        _check_bits_group(bits, group_size)
        if act_bits not in (None, 8):
            raise ValueError(f"act_bits must be None or 8, got {act_bits}")
        self.act_bits = act_bits
        if dtype not in _SZ_DTYPES:
            raise ValueError(f"dtype must be one of {_SZ_DTYPES}")
        if in_features % group_size != 0:
            raise ValueError(f"in_features={in_features} is not a multiple of group_size={group_size}")
        self.in_features, self.out_features = in_features, out_features
        self.bits, self.group_size, self.dtype = bits, group_size, dtype
        self._call = None            # prepared eager call (made on first use)
        G = in_features // group_size
        self.register_buffer("packed", torch.zeros((out_features, in_features * bits // 8),
                                                   dtype=torch.uint8, device=device))
        self.register_buffer("scales", torch.zeros((out_features, G), dtype=dtype, device=device))
        self.register_buffer("zeros", torch.zeros((out_features, G), dtype=dtype, device=device))
        if bias:
            self.register_buffer("bias", torch.zeros((out_features,), dtype=dtype, device=device))
        else:
            self.bias = None

    @torch.no_grad()
    def set_weight(self, weight: torch.Tensor, bias: Optional[torch.Tensor] = None) -> "LowbitLinear":
        """Quantize a float ``weight[N, K]`` (on the GPU) into this module."""
        if tuple(weight.shape) != (self.out_features, self.in_features):
            raise ValueError(f"weight must be [{self.out_features}, {self.in_features}]")
        packed, scales, zeros = torch.ops.lowbit.quantize_pack(weight.detach(), self.bits,
                                                               self.group_size, self.dtype)
        self.packed.copy_(packed)
        self.scales.copy_(scales)
        self.zeros.copy_(zeros)
        if self.bias is not None:
            if bias is None:
                self.bias.zero_()
            else:
                self.bias.copy_(bias.detach().to(self.dtype))
        return self

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, bits: int, group_size: int,
                    dtype: Optional[torch.dtype] = None,
                    act_bits: Optional[int] = None) -> "LowbitLinear":
        """Quantize ``lin`` on the fly (its weight must live on the GPU)."""
        dt = dtype or (lin.weight.dtype if lin.weight.dtype in _SZ_DTYPES else torch.float16)
        m = cls(lin.in_features, lin.out_features, bits, group_size, bias=lin.bias is not None,
                dtype=dt, device=lin.weight.device, act_bits=act_bits)
        return m.set_weight(lin.weight, lin.bias)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.act_bits == 8:
            return torch.ops.lowbit.linear_a8(x, self.packed, self.scales, self.zeros, self.bias,
                                              self.bits, self.group_size)
        # Traced (torch.compile), autograd and non-GPU (e.g. meta) calls go
        # through the registered op; plain eager GPU calls take the prepared
        # call, which validated the weights once (buffers replaced by .to()
        # and the like make a new one).
        if (not x.is_cuda or torch.compiler.is_compiling()
                or (x.requires_grad and torch.is_grad_enabled())):
            return torch.ops.lowbit.linear(x, self.packed, self.scales, self.zeros, self.bias,
                                           self.bits, self.group_size)
        b = self._buffers
        call = self._call
        if (call is None or call._keep[0] is not b["packed"] or call._keep[1] is not b["scales"]
                or call._keep[2] is not b["zeros"] or call._keep[3] is not b.get("bias")):
            call = _lb.PreparedLinear(b["packed"], b["scales"], b["zeros"], b.get("bias"),
                                      self.bits, self.group_size)
            self._call = call
        if x.dim() == 2:
            return call(x.contiguous())
        y = call(x.reshape(-1, self.in_features).contiguous())
        return y.reshape(*x.shape[:-1], self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, bits={self.bits}, "
                f"group_size={self.group_size}, dtype={self.dtype}, bias={self.bias is not None}"
                + ("" if self.act_bits is None else f", act_bits={self.act_bits}"))


def quantize_linears(model: torch.nn.Module, bits: int, group_size: int,
                     dtype: Optional[torch.dtype] = None,
                     filter_fn: Optional[Callable[[torch.nn.Module, str], bool]] = None,
                     act_bits: Optional[int] = None) -> torch.nn.Module:
    """Replace every ``nn.Linear`` of ``model`` (in place) by a LowbitLinear.

    ``filter_fn(module, qualified_name)`` may exclude layers; layers whose
    in_features is not a multiple of ``group_size`` are left as they are.
    ``act_bits=8`` makes every swapped layer quantize its activations too.
    """
    for name, child in list(model.named_children()):
        _swap(model, name, child, name, bits, group_size, dtype, filter_fn, act_bits)
    return model


def _swap(parent, name, child, qual, bits, group_size, dtype, filter_fn, act_bits):
    if isinstance(child, torch.nn.Linear):
        if child.in_features % group_size == 0 and (filter_fn is None or filter_fn(child, qual)):
            setattr(parent, name, LowbitLinear.from_linear(child, bits, group_size, dtype, act_bits))
        return
    for n, c in list(child.named_children()):
        _swap(child, n, c, f"{qual}.{n}", bits, group_size, dtype, filter_fn, act_bits)
