"""Binding of the benchmark's measurement probes (liblowbit_probe.so, C ABI in
include/lowbit_probe.h): a plain streaming read and a dependent-load chain,
used to report the decode kernel against the single-launch floor of the
device.  Not part of the layer; argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import lowbit as _lb

_PKG = os.path.dirname(os.path.abspath(__file__))
EXPORTED_SYMBOLS = ("lowbit_probe_stream_read", "lowbit_probe_chase", "lowbit_probe_last_error")
_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.path.join(_PKG, "liblowbit_probe.so")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"probe library not built: {path} is missing "
                           f"(build it with __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    c_i64, c_sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.lowbit_probe_stream_read.restype = ctypes.c_int
    lib.lowbit_probe_stream_read.argtypes = [vp, c_sz, ctypes.c_int, vp, vp]
    lib.lowbit_probe_chase.restype = ctypes.c_int
    lib.lowbit_probe_chase.argtypes = [vp, c_i64, ctypes.c_int, ctypes.c_uint32, vp, vp]
    lib.lowbit_probe_last_error.restype = ctypes.c_char_p
    lib.lowbit_probe_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != _lb.LOWBIT_OK:
        raise _lb.LowbitError(status, func, load().lowbit_probe_last_error().decode(errors="replace"))


def stream_read(src: torch.Tensor, nbytes: int, loads_per_thread: int, sink: torch.Tensor,
                stream=None) -> None:
    """Read the first nbytes of src (device) with plain 16-byte loads in one launch."""
    lib = load()
    _lb._require_cuda(src, sink)
    _lb._expect(nbytes <= src.numel() * src.element_size(), "nbytes exceeds src")
    _lb._expect(sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 1, "sink: one 32-bit word")
    with torch.cuda.device(src.device):
        st = lib.lowbit_probe_stream_read(src.data_ptr(), nbytes, loads_per_thread, sink.data_ptr(),
                                          _lb._stream_handle(src.device, stream))
    _check(st, "lowbit_probe_stream_read")


def chase(chain: torch.Tensor, hops: int, start: int, out: torch.Tensor, stream=None) -> None:
    """Follow hops dependent links i <- chain[i] (int32/uint32 device array) from start."""
    lib = load()
    _lb._require_cuda(chain, out)
    _lb._expect(chain.dtype in (torch.int32, torch.uint32) and chain.is_contiguous(), "chain: 32-bit, contiguous")
    _lb._expect(out.dtype in (torch.int32, torch.uint32) and out.numel() >= 1, "out: one 32-bit word")
    with torch.cuda.device(chain.device):
        st = lib.lowbit_probe_chase(chain.data_ptr(), chain.numel(), hops, start, out.data_ptr(),
                                    _lb._stream_handle(chain.device, stream))
    _check(st, "lowbit_probe_chase")
