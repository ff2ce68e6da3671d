"""Python binding of the C ABI in include/lowbit.h (ctypes, argument marshalling only).

Every step of the computation runs in the HIP library liblowbit.so; this module
only turns torch tensors into device pointers and sizes, allocates outputs with
torch when the caller does not pass them, and raises LowbitError on a non-OK
status.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "liblowbit.so"

LOWBIT_OK = 0
STATUS_NAMES = {
    0: "LOWBIT_OK", 1: "LOWBIT_ERR_INVALID_ARG", 2: "LOWBIT_ERR_UNSUPPORTED",
    3: "LOWBIT_ERR_MISALIGNED", 4: "LOWBIT_ERR_NONFINITE", 5: "LOWBIT_ERR_RANGE",
    6: "LOWBIT_ERR_WORKSPACE", 7: "LOWBIT_ERR_HIP",
}
LOWBIT_F32, LOWBIT_F16, LOWBIT_BF16 = 0, 1, 2
PATH_AUTO, PATH_QMV, PATH_QMM = 0, 1, 2
_DTYPE_ENUM = {torch.float32: LOWBIT_F32, torch.float16: LOWBIT_F16, torch.bfloat16: LOWBIT_BF16}
_ENUM_DTYPE = {v: k for k, v in _DTYPE_ENUM.items()}

EXPORTED_SYMBOLS = (
    "lowbit_abi_version", "lowbit_packed_bytes", "lowbit_num_groups", "lowbit_quantize_pack",
    "lowbit_linear_workspace_bytes", "lowbit_linear", "lowbit_linear_path", "lowbit_linear_multi",
    "lowbit_status_string", "lowbit_last_error", "lowbit_linear_noalloc", "lowbit_set_tuning",
    "lowbit_quantize_act_i8", "lowbit_linear_a8",
)
ABI_VERSION = 3
# schedule overrides (include/lowbit_tuning.h)
TUNE_KEYS = {"qmv_block": 0, "qmv_variant": 1, "qmm_blocks": 2, "qmm_mtt": 3, "qmm_kgroups": 4,
             "qmm_nt": 5, "qmm_waves": 6, "qmm_rgroups": 7, "qmm_small_m": 8,
             "a8_mtt": 9, "a8_nt": 10}
MAX_MULTI = 8   # LOWBIT_MAX_MULTI


class LinearDesc(ctypes.Structure):
    """struct lowbit_linear_desc"""
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class LowbitError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{func}: {self.status_name}: {detail}")


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.environ.get("LOWBIT_LIBRARY", os.path.join(_PKG, _LIB_NAME))


def load() -> ctypes.CDLL:
    """Load liblowbit.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           f"(build it with __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    c_i64, c_sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.lowbit_abi_version.restype = ctypes.c_int
    lib.lowbit_abi_version.argtypes = []
    lib.lowbit_packed_bytes.restype = c_sz
    lib.lowbit_packed_bytes.argtypes = [ctypes.c_int, c_i64, c_i64]
    lib.lowbit_num_groups.restype = c_i64
    lib.lowbit_num_groups.argtypes = [c_i64, ctypes.c_int]
    lib.lowbit_quantize_pack.restype = ctypes.c_int
    lib.lowbit_quantize_pack.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, c_i64, c_i64,
                                         ctypes.c_int, vp, vp, vp, vp, vp]
    lib.lowbit_linear_workspace_bytes.restype = c_sz
    lib.lowbit_linear_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, c_i64, c_i64, c_i64,
                                                  ctypes.c_int]
    lin = [vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, c_i64, c_i64, c_i64,
           vp, c_sz]
    lib.lowbit_linear.restype = ctypes.c_int
    lib.lowbit_linear.argtypes = lin + [vp]
    lib.lowbit_linear_path.restype = ctypes.c_int
    lib.lowbit_linear_path.argtypes = lin + [ctypes.c_int, vp]
    lib.lowbit_linear_noalloc.restype = ctypes.c_int
    lib.lowbit_linear_noalloc.argtypes = lin[:12] + [vp]
    lib.lowbit_linear_multi.restype = ctypes.c_int
    lib.lowbit_linear_multi.argtypes = [ctypes.POINTER(LinearDesc), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, c_i64, vp]
    lib.lowbit_status_string.restype = ctypes.c_char_p
    lib.lowbit_status_string.argtypes = [ctypes.c_int]
    lib.lowbit_last_error.restype = ctypes.c_char_p
    lib.lowbit_last_error.argtypes = []
    lib.lowbit_set_tuning.restype = ctypes.c_int
    lib.lowbit_set_tuning.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.lowbit_quantize_act_i8.restype = ctypes.c_int
    lib.lowbit_quantize_act_i8.argtypes = [vp, ctypes.c_int, c_i64, c_i64, vp, vp, vp]
    lib.lowbit_linear_a8.restype = ctypes.c_int
    lib.lowbit_linear_a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, c_i64, c_i64, c_i64, vp]
    if lib.lowbit_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.lowbit_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it with __graft_entry__.build()")
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != LOWBIT_OK:
        detail = load().lowbit_last_error().decode(errors="replace")
        raise LowbitError(status, func, detail)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(device: torch.device, stream) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if device.type != "cuda":
        return None
    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(*tensors: Optional[torch.Tensor]) -> None:
    devices = set()
    for t in tensors:
        if t is not None and t.device.type != "cuda":
            raise ValueError("lowbit tensors must live in GPU memory (device 'cuda')")
        if t is not None and not t.is_contiguous():
            raise ValueError("lowbit tensors must be contiguous")
        if t is not None:
            devices.add(t.device)
    if len(devices) > 1:
        raise ValueError(f"lowbit tensors must all be on one device, got {sorted(map(str, devices))}")


def _expect(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


_GROUPS = (32, 64, 128, 256)


# The C interface takes raw pointers and cannot see buffer sizes or dtypes;
# these checks keep every kernel access inside the tensors passed here.
# (Messages are formatted only on failure: the checks run on every call.)
def _check_weight_tensors(packed, scales, zeros, N: int, K: int, bits: int, group: int,
                          sz_dtype: torch.dtype) -> None:
    if not 1 <= bits <= 7:
        raise ValueError(f"bits must be in 1..7, got {bits}")
    if group not in _GROUPS:
        raise ValueError(f"group must be 32, 64, 128 or 256, got {group}")
    if K % group:
        raise ValueError(f"K={K} is not a multiple of group={group}")
    if packed.dtype != torch.uint8:
        raise ValueError("packed must be uint8")
    if packed.numel() != N * K * bits // 8:
        raise ValueError(f"packed holds {packed.numel()} bytes, expected N*K*bits/8 = {N * K * bits // 8}")
    G = K // group
    for name, t in (("scales", scales), ("zeros", zeros)):
        shp = t.shape
        if len(shp) != 2 or shp[0] != N or shp[1] != G:
            raise ValueError(f"{name} must be [{N}, {G}], got {tuple(shp)}")
        if t.dtype != sz_dtype:
            raise ValueError(f"{name} must be {sz_dtype}, got {t.dtype}")


def _check_linear_tensors(x, packed, scales, zeros, bias, y, bits: int, group: int) -> Tuple[int, int, int]:
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    dt = x.dtype
    if dt not in _DTYPE_ENUM:
        raise ValueError(f"x dtype {dt} is not float32, float16 or bfloat16")
    if scales.dim() != 2:
        raise ValueError("scales must be 2-D [N, K/group]")
    M, K = x.shape
    N = scales.shape[0]
    _check_weight_tensors(packed, scales, zeros, N, K, bits, group, dt)
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or bias.dtype != dt):
        raise ValueError(f"bias must be [{N}] of {dt}")
    if y is not None and (y.dim() != 2 or y.shape[0] != M or y.shape[1] != N or y.dtype != dt):
        raise ValueError(f"y must be [{M}, {N}] of {dt}")
    return M, N, K


# ---------------------------------------------------------------- C calls --

def lowbit_abi_version() -> int:
    return load().lowbit_abi_version()


def lowbit_packed_bytes(bits: int, N: int, K: int) -> int:
    return load().lowbit_packed_bytes(bits, N, K)


def lowbit_num_groups(K: int, group: int) -> int:
    return load().lowbit_num_groups(K, group)


def lowbit_linear_workspace_bytes(bits: int, group: int, M: int, N: int, K: int,
                                  act_dtype: torch.dtype) -> int:
    return load().lowbit_linear_workspace_bytes(bits, group, M, N, K, _DTYPE_ENUM[act_dtype])


def lowbit_status_string(status: int) -> str:
    return load().lowbit_status_string(status).decode()


def lowbit_last_error() -> str:
    return load().lowbit_last_error().decode(errors="replace")


def lowbit_quantize_pack(w: torch.Tensor, bits: int, group: int, sz_dtype: torch.dtype,
                         want_codes: bool = False, out: Optional[Tuple] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                               Optional[torch.Tensor]]:
    """Quantize w[N, K] (fp32, or fp16 / bf16 taken exactly as fp32) on the GPU.
    Returns (packed, scales, zeros, codes|None).

    `out` may give preallocated (packed, scales, zeros, codes) tensors.
    """
    lib = load()
    _expect(w.dim() == 2, "w must be 2-D [N, K]")
    _expect(w.dtype in _DTYPE_ENUM, f"w must be float32, float16 or bfloat16, got {w.dtype}")
    _expect(sz_dtype in _DTYPE_ENUM, f"sz_dtype {sz_dtype} is not float32, float16 or bfloat16")
    N, K = w.shape
    if out is None:
        nbytes = lib.lowbit_packed_bytes(bits, N, K)
        G = lib.lowbit_num_groups(K, group)
        dev = w.device
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)[:nbytes].view(N, -1) \
            if nbytes else torch.empty(0, dtype=torch.uint8, device=dev)
        scales = torch.empty((N, max(G, 0)), dtype=sz_dtype, device=dev)
        zeros = torch.empty((N, max(G, 0)), dtype=sz_dtype, device=dev)
        codes = torch.empty((N, K), dtype=torch.uint8, device=dev) if want_codes else None
    else:
        packed, scales, zeros, codes = out
    if bits in range(1, 8) and group in (32, 64, 128, 256) and K % group == 0:
        _check_weight_tensors(packed, scales, zeros, N, K, bits, group, sz_dtype)
    if codes is not None:
        _expect(tuple(codes.shape) == (N, K) and codes.dtype == torch.uint8, f"codes must be [{N}, {K}] uint8")
    _require_cuda(w, packed, scales, zeros, codes)
    with torch.cuda.device(w.device):
        st = lib.lowbit_quantize_pack(_ptr(w), _DTYPE_ENUM[w.dtype], bits, group, N, K,
                                      _DTYPE_ENUM[sz_dtype], _ptr(scales),
                                      _ptr(zeros), _ptr(packed), _ptr(codes),
                                      _stream_handle(w.device, stream))
    _check(st, "lowbit_quantize_pack")
    return packed, scales, zeros, codes


# Workspaces kept per (device, stream): calls on one stream run in order, so
# they never use the same workspace at the same time.  A buffer handed out
# once is never freed: a HIP graph captured over a call keeps its address and
# writes to it on every replay, so when a larger workspace is needed the old
# one is retired (kept alive), not released.  Sizes grow by powers of two, so
# the retired buffers add up to less than the current one.
_workspaces = {}
_retired_workspaces = []


def cached_workspace(device: torch.device, stream_handle, nbytes: int) -> Optional[torch.Tensor]:
    """A device buffer of at least nbytes reserved for calls on this stream."""
    if nbytes <= 0:
        return None
    key = (device.index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired_workspaces.append(ws)
        size = 1 << max(20, (nbytes - 1).bit_length())
        ws = torch.empty(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def lowbit_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                  bias: Optional[torch.Tensor], bits: int, group: int,
                  y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  path: Optional[int] = None, stream=None) -> torch.Tensor:
    """y[M, N] = x[M, K] . dequant(packed, scales, zeros)^T (+ bias), on the GPU.

    Without an explicit `workspace`, a buffer cached for this device and
    stream is used (calls on one stream run in order, so they never share it
    concurrently).
    """
    lib = load()
    M, N, K = _check_linear_tensors(x, packed, scales, zeros, bias, y, bits, group)
    if workspace is not None:
        _expect(workspace.dtype == torch.uint8, "workspace must be uint8")
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    s = _stream_handle(x.device, stream)
    if workspace is None and M > 0 and x.dtype in _DTYPE_ENUM:
        need = lib.lowbit_linear_workspace_bytes(bits, group, M, N, K, _DTYPE_ENUM[x.dtype])
        workspace = cached_workspace(x.device, s, need)
    _require_cuda(x, packed, scales, zeros, bias, y, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _DTYPE_ENUM[x.dtype], _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(bias),
            _ptr(y), bits, group, M, N, K, _ptr(workspace), ws_bytes)
    with torch.cuda.device(x.device):
        if path is None:
            st = lib.lowbit_linear(*args, s)
        else:
            st = lib.lowbit_linear_path(*args, int(path), s)
    _check(st, "lowbit_linear" if path is None else "lowbit_linear_path")
    return y


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _fastcall_module():
    """The compiled argument-marshalling module for eager calls, or None
    (then PreparedLinear passes ctypes values; both call the same entry)."""
    try:
        from bit_groupwise_weight_amd import _lowbit_fastcall
        return _lowbit_fastcall
    except ImportError:
        return None


class PreparedLinear:
    """One layer's weights bound to lowbit_linear once, for eager calls.

    The weight tensors (packed, scales, zeros, bias) are validated when the
    object is made and their device pointers kept (with references to the
    tensors); a call then checks only x and y, takes the current stream's raw
    handle and the workspace cached for (M, stream), and makes the one C call.
    The result is that of lowbit_linear with the same arguments.  Rebuild the
    object if the weight tensors are replaced (in-place updates keep it valid).
    """

    __slots__ = ("N", "K", "bits", "group", "dtype", "act", "device", "dev_index", "_ptrs",
                 "_keep", "_fn", "_ws", "_const", "_one_device", "_fc", "_bound")

    def __init__(self, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 bias: Optional[torch.Tensor], bits: int, group: int):
        lib = load()
        _expect(scales.dim() == 2, "scales must be 2-D [N, K/group]")
        dt = scales.dtype
        _expect(dt in _DTYPE_ENUM, f"scales dtype {dt} is not float32, float16 or bfloat16")
        N, G = scales.shape
        K = G * group
        _check_weight_tensors(packed, scales, zeros, N, K, bits, group, dt)
        if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or bias.dtype != dt):
            raise ValueError(f"bias must be [{N}] of {dt}")
        _require_cuda(packed, scales, zeros, bias)
        self.N, self.K, self.bits, self.group = N, K, bits, group
        self.dtype, self.act = dt, _DTYPE_ENUM[dt]
        self.device = packed.device
        self.dev_index = packed.get_device()
        self._one_device = torch.cuda.device_count() == 1   # then no device switch is ever needed
        self._ptrs = (packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), _ptr(bias))
        self._keep = (packed, scales, zeros, bias)
        # the same entry point without argument types: every argument is
        # passed as a ready ctypes value (the ones fixed for this layer are
        # made here), which skips the per-argument conversion of a call
        self._fn = type(lib.lowbit_linear)(("lowbit_linear", lib))
        self._fn.restype = ctypes.c_int
        vp, ci = ctypes.c_void_p, ctypes.c_int
        self._const = (ci(self.act), vp(self._ptrs[0]), vp(self._ptrs[1]), vp(self._ptrs[2]),
                       vp(self._ptrs[3]), ci(bits), ci(group), ctypes.c_int64(N), ctypes.c_int64(K))
        # with the compiled marshalling module, the fixed arguments are bound
        # once in C and a call passes seven ints
        self._fc = _fastcall_module()
        self._bound = None
        if self._fc is not None:
            fn = ctypes.cast(lib.lowbit_linear, ctypes.c_void_p).value
            self._bound = self._fc.bind(fn, self.act, self._ptrs[0], self._ptrs[1], self._ptrs[2],
                                        self._ptrs[3], bits, group, N, K)
        self._ws = {}

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """y[M, N] = x[M, K] . dequant(W)^T (+ bias) for this layer."""
        if (x.dtype is not self.dtype or x.dim() != 2 or x.shape[1] != self.K
                or x.get_device() != self.dev_index or not x.is_contiguous()):
            raise ValueError(f"x must be a contiguous [M, {self.K}] {self.dtype} tensor on {self.device}")
        M = x.shape[0]
        N = self.N
        if y is None:
            y = torch.empty((M, N), dtype=self.dtype, device=self.device)
        elif (y.dtype is not self.dtype or y.dim() != 2 or y.shape[0] != M or y.shape[1] != N
              or y.get_device() != self.dev_index or not y.is_contiguous()):
            raise ValueError(f"y must be a contiguous [{M}, {N}] {self.dtype} tensor on {self.device}")
        if stream is not None:
            s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        elif _raw_stream is not None:
            s = _raw_stream(self.dev_index)
        else:
            s = torch.cuda.current_stream(self.device).cuda_stream
        key = (M, s)
        tail = self._ws.get(key)
        if tail is None:
            need = load().lowbit_linear_workspace_bytes(self.bits, self.group, M, N, self.K, self.act)
            buf = cached_workspace(self.device, s, need) if M > 0 else None
            ws_ptr, ws_bytes = (0, 0) if buf is None else (buf.data_ptr(), buf.numel())
            tail = (ws_ptr, ws_bytes, ctypes.c_int64(M), ctypes.c_void_p(ws_ptr or None),
                    ctypes.c_size_t(ws_bytes), ctypes.c_void_p(s))
            self._ws[key] = tail
        same_device = self._one_device or torch.cuda.current_device() == self.dev_index
        if self._bound is not None and same_device:
            st = self._fc.call(self._bound, x.data_ptr(), y.data_ptr(), M, tail[0], tail[1], s)
        else:
            act, pk, sp, zp, bp, bits, group, n, k = self._const
            m, wp, wb, sh = tail[2:]
            args = (ctypes.c_void_p(x.data_ptr()), act, pk, sp, zp, bp, ctypes.c_void_p(y.data_ptr()),
                    bits, group, m, n, k, wp, wb, sh)
            if same_device:
                st = self._fn(*args)
            else:
                with torch.cuda.device(self.device):
                    st = self._fn(*args)
        if st != LOWBIT_OK:
            _check(st, "lowbit_linear")
        return y


def lowbit_linear_noalloc(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                          zeros: torch.Tensor, bias: Optional[torch.Tensor], bits: int, group: int,
                          y: torch.Tensor, stream=None) -> torch.Tensor:
    """lowbit_linear that allocates nothing: `y` is required, and the split-K
    partials of the MFMA schedule live in the library's own device array
    (calls that overlap in time on one GPU race; calls on one stream are safe)."""
    lib = load()
    _expect(y is not None, "y is required (this call allocates nothing)")
    M, N, K = _check_linear_tensors(x, packed, scales, zeros, bias, y, bits, group)
    _require_cuda(x, packed, scales, zeros, bias, y)
    with torch.cuda.device(x.device):
        st = lib.lowbit_linear_noalloc(_ptr(x), _DTYPE_ENUM[x.dtype], _ptr(packed), _ptr(scales),
                                       _ptr(zeros), _ptr(bias), _ptr(y), bits, group, M, N, K,
                                       _stream_handle(x.device, stream))
    _check(st, "lowbit_linear_noalloc")
    return y


def lowbit_quantize_act_i8(x: torch.Tensor, xq: Optional[torch.Tensor] = None,
                           ascale: Optional[torch.Tensor] = None, stream=None):
    """Per-row symmetric int8 codes of x[M, K] and their fp32 scales (on the GPU).

    Returns (xq int8 [M, K], ascale float32 [M]); a row holding a NaN or an
    infinity gets a NaN scale and codes 0."""
    lib = load()
    _expect(x.dim() == 2, "x must be 2-D [M, K]")
    _expect(x.dtype in _DTYPE_ENUM, f"x dtype {x.dtype} is not float32, float16 or bfloat16")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if ascale is None:
        ascale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _expect(xq.dtype == torch.int8 and tuple(xq.shape) == (M, K), f"xq must be int8 [{M}, {K}]")
    _expect(ascale.dtype == torch.float32 and tuple(ascale.shape) == (M,),
            f"ascale must be float32 [{M}]")
    _require_cuda(x, xq, ascale)
    with torch.cuda.device(x.device):
        st = lib.lowbit_quantize_act_i8(_ptr(x), _DTYPE_ENUM[x.dtype], M, K, _ptr(xq), _ptr(ascale),
                                        _stream_handle(x.device, stream))
    _check(st, "lowbit_quantize_act_i8")
    return xq, ascale


def lowbit_linear_a8(xq: torch.Tensor, ascale: torch.Tensor, packed: torch.Tensor,
                     scales: torch.Tensor, zeros: torch.Tensor, bias: Optional[torch.Tensor],
                     bits: int, group: int, y: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """y = diag(ascale) . xq . dequant(packed, scales, zeros)^T (+ bias) on the
    int8 matrix cores; y, bias, scales and zeros share one dtype."""
    lib = load()
    _expect(xq.dim() == 2 and xq.dtype == torch.int8, "xq must be int8 [M, K]")
    _expect(scales.dim() == 2, "scales must be 2-D [N, K/group]")
    M, K = xq.shape
    N = scales.shape[0]
    dt = scales.dtype
    _expect(dt in _DTYPE_ENUM, f"scales dtype {dt} is not float32, float16 or bfloat16")
    _check_weight_tensors(packed, scales, zeros, N, K, bits, group, dt)
    _expect(ascale.dtype == torch.float32 and tuple(ascale.shape) == (M,),
            f"ascale must be float32 [{M}]")
    if bias is not None:
        _expect(bias.dim() == 1 and bias.shape[0] == N and bias.dtype == dt, f"bias must be [{N}] of {dt}")
    if y is None:
        y = torch.empty((M, N), dtype=dt, device=xq.device)
    _expect(y.dim() == 2 and tuple(y.shape) == (M, N) and y.dtype == dt, f"y must be [{M}, {N}] of {dt}")
    _require_cuda(xq, ascale, packed, scales, zeros, bias, y)
    with torch.cuda.device(xq.device):
        st = lib.lowbit_linear_a8(_ptr(xq), _ptr(ascale), _ptr(packed), _ptr(scales), _ptr(zeros),
                                  _ptr(bias), _ptr(y), _DTYPE_ENUM[dt], bits, group, M, N, K,
                                  _stream_handle(xq.device, stream))
    _check(st, "lowbit_linear_a8")
    return y


def lowbit_linear_multi(items, bits: int, group: int, stream=None):
    """Several linears in one launch: items are (x, packed, scales, zeros, bias, y)
    tuples sharing bits, group, x's dtype and M; y may be None (allocated).
    Returns the list of outputs."""
    lib = load()
    if not items:
        return []
    if len(items) > MAX_MULTI:
        raise ValueError(f"at most {MAX_MULTI} linears per call")
    x0 = items[0][0]
    M, dtype = x0.shape[0], x0.dtype
    descs = (LinearDesc * len(items))()
    outs = []
    shapes = []
    for x, packed, scales, zeros, bias, y in items:      # every item is checked before any runs
        _expect(x.dim() == 2 and x.shape[0] == M and x.dtype == dtype,
                "every x must be 2-D with the same M and dtype")
        shapes.append(_check_linear_tensors(x, packed, scales, zeros, bias, y, bits, group))
    for i, ((x, packed, scales, zeros, bias, y), (_, N, K)) in enumerate(zip(items, shapes)):
        if y is None:
            y = torch.empty((M, N), dtype=dtype, device=x.device)
        _require_cuda(x0, x, packed, scales, zeros, bias, y)
        descs[i] = LinearDesc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(bias), _ptr(y), N, K)
        outs.append(y)
    with torch.cuda.device(x0.device):
        st = lib.lowbit_linear_multi(descs, len(items), _DTYPE_ENUM[dtype], bits, group, M,
                                     _stream_handle(x0.device, stream))
    _check(st, "lowbit_linear_multi")
    return outs


# ----------------------------------------------------------------- tuning --

def lowbit_set_tuning(key: str, value: int) -> None:
    """Set (value > 0) or clear (0) a schedule override (tests and benchmarks)."""
    _check(load().lowbit_set_tuning(TUNE_KEYS[key], int(value)), "lowbit_set_tuning")


class tuning:
    """Context manager: schedule overrides for the calls inside it, e.g.
    `with lowbit.tuning(qmm_nt=1, qmm_kgroups=2): ...`; cleared on exit."""

    def __init__(self, **overrides: int):
        self.overrides = overrides

    def __enter__(self):
        for k, v in self.overrides.items():
            lowbit_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k in self.overrides:
            lowbit_set_tuning(k, 0)
        return False
