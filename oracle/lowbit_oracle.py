"""CPU oracle for the groupwise weight-only low-bit linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP library.

What it computes (plain numpy, slow and obvious):

  quantize  -- per output row n and per group g of `group` consecutive
               K-elements: an asymmetric min/max fit giving one scale and one
               zero per (row, group), stored N x num_groups.  Codes are
               unsigned b-bit integers in [0, 2^b - 1].
  pack      -- codes of one row laid out as one contiguous bit stream:
               bit j of code k sits at stream bit k*b + j, stream bit p lives in
               byte p >> 3 at bit p & 7 (least significant bit first), so codes
               cross byte boundaries when b does not divide 8.
  linear    -- y[m, n] = sum_k x[m, k] * (s[n, k/group] * q[n, k] + z[n, k/group])
               (+ bias[n]) in float64, and the tolerance scale
               A[m, n] = sum_k |x[m, k] * w[n, k]| with w the dequantized weight.

Sources (cited by page title and section):
  * "Add torchao mps ops" -- the linear:afpwx description: weight-only,
    groupwise, bit widths 1..7, group sizes 32/64/128/256.
  * "metal lowbit kernels: qmv_fast optimization", Summary -- scales and zeros
    are shaped N x num_groups, as the quantize function produces them; bits of
    3/5/6/7-bit codes are stored contiguously, moving on to the next byte when
    the current byte is full.
  * "Revamp int4 MPS support in torchao" -- bias must be supported.

Readings where the pages are silent (each one is listed in the design notes):
  R1  dequantization is w = s*q + z, z a real offset in the same dtype as s.
  R2  asymmetric min/max: s = (max - min) / (2^b - 1), z = min.
  R3  codes round half to even.
  R4  a constant group (max == min) gets s = 0 and q = 0; it reconstructs to z.
  R5  s and z are stored in the activation dtype (fp32, fp16 or bf16).
  R6  s and z are rounded to their storage dtype first, and codes are computed
      from the stored values: q = clamp(rint((w - z_st) / s_st), 0, 2^b - 1).
  R7  the fp32 steps are single IEEE operations in the order written: a
      subtract, then a correctly rounded divide; no fused multiply-add.
  R8  packing is least-significant-bit first inside each byte.
  R9  1-, 2- and 4-bit codes follow the same rule (they never straddle).
  R10 each row's byte string has K*b/8 bytes, no padding.
  R11 s and z are indexed [n][k // group], row-major.
  R12 W arrives as fp32.
  R22 signed zeros compare equal in the min/max scan; a zero minimum or maximum
      is taken as +0.

Activation-quantized variant (the "-qmode 8da4w -G 32" export mode of
"[MPS] Add support for Int4 groupwise quantization": 8-bit dynamic
activations with 4-bit weights in groups of 32; the page names the mode and
nothing of its arithmetic, so these readings fix it):
  R30 each activation row m is quantized on the fly to signed 8-bit codes with
      one fp32 scale: a_m = max_k |x[m, k]| / 127 (an fp32 correctly rounded
      divide), xq[m, k] = clamp(rint_half_even(x[m, k] / a_m), -127, 127) with
      the divide in fp32 (symmetric: no zero point, -128 unused).
  R31 a row whose a_m is 0 (all zeros, or a maximum so small that the divide
      underflows) gets all codes 0.
  R32 a row holding a NaN or an infinity gets a_m = NaN and all codes 0, so
      its outputs are NaN.
  R33 the weights keep this module's format (R1-R11, any width and group);
      y[m, n] = sum_k (a_m * xq[m, k]) * w[n, k] (+ bias[n]): the integer
      group sums sum xq*q and sum xq are exact, and the tolerance of the
      weight-only linear applies with x replaced by a_m * xq.

Parity status: every function below is pinned by tests that do not reuse its
own formula (golden packing vectors derived by hand, a big-integer bit-stream
formulation, a pure-Python bit reader, exact-grid / tie / constant-group closed
forms, one-hot and group-ones inputs, exact integer and exact rational matmuls,
and torch's bfloat16 cast).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


class OracleError(Exception):
    """Base class for rejected inputs."""


class NonFiniteInput(OracleError):
    pass


class RangeError(OracleError):
    pass


SUPPORTED_BITS = (1, 2, 3, 4, 5, 6, 7)
SUPPORTED_GROUPS = (32, 64, 128, 256)
STORAGE_DTYPES = ("f32", "f16", "bf16")


# ------------------------------------------------------------ storage casts --

def round_f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 with round-to-nearest-even, returned as uint16 bit patterns.

    bfloat16 is the top half of an fp32 word.  Rounding to nearest even on the
    dropped 16 bits: add 0x7FFF plus the lowest kept bit, then truncate.  NaNs
    are kept quiet NaNs.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = np.isnan(np.asarray(a, dtype=np.float32))
    out = np.where(is_nan, (u >> np.uint64(16)) | np.uint64(0x0040), rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def round_to_storage(a32: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to the storage dtype (nearest even).

    Returns (values as fp32, raw bit patterns: uint32 for f32, uint16 otherwise).
    """
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32.copy(), a32.view(np.uint32).copy()
    if dtype == "f16":
        with np.errstate(over="ignore"):
            h = a32.astype(np.float16)          # IEEE binary16, nearest even
        return h.astype(np.float32), h.view(np.uint16).copy()
    if dtype == "bf16":
        bits = round_f32_to_bf16_bits(a32)
        return bf16_bits_to_f32(bits), bits
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------- quantize --

def check_params(bits: int, group: int, K: int) -> None:
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}, got {bits}")
    if group not in SUPPORTED_GROUPS:
        raise ValueError(f"group must be one of {SUPPORTED_GROUPS}, got {group}")
    if K <= 0 or K % group != 0:
        raise ValueError(f"K={K} must be a positive multiple of group={group}")


def quantize(W: np.ndarray, bits: int, group: int, sz_dtype: str):
    """Asymmetric per-(row, group) min/max quantization of W[N, K] (fp32).

    Follows R2-R7 and R22.  Returns a dict with
      q      uint8  [N, K]      codes in [0, 2^b - 1]
      s, z   fp32   [N, K/group] stored scale / zero values (exact in sz_dtype)
      s_bits, z_bits             their raw bit patterns in sz_dtype
    Raises NonFiniteInput for a non-finite weight and RangeError when a stored
    scale or zero is not finite.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    check_params(bits, group, K)
    if not np.all(np.isfinite(W)):
        raise NonFiniteInput("weight contains a non-finite value")
    G = K // group
    Wg = W.reshape(N, G, group)
    qmax = np.float32((1 << bits) - 1)

    mn = Wg.min(axis=2)                       # exact
    mx = Wg.max(axis=2)
    mn = np.where(mn == 0, np.float32(0.0), mn).astype(np.float32)   # R22
    mx = np.where(mx == 0, np.float32(0.0), mx).astype(np.float32)

    with np.errstate(over="ignore"):
        s32 = (mx - mn) / qmax                # fp32 subtract, then fp32 divide
    z32 = mn

    s_st, s_bits = round_to_storage(s32, sz_dtype)
    z_st, z_bits = round_to_storage(z32, sz_dtype)
    if not (np.all(np.isfinite(s_st)) and np.all(np.isfinite(z_st))):
        raise RangeError("a scale or zero is not finite in the storage dtype")

    s_b = s_st[:, :, None]
    z_b = z_st[:, :, None]
    nonzero = s_b != 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = (Wg - z_b) / np.where(nonzero, s_b, np.float32(1.0))    # fp32, R7
    t = t.astype(np.float32)
    q = np.clip(np.rint(t), np.float32(0.0), qmax)                  # R3: half to even
    q = np.where(nonzero, q, np.float32(0.0))                       # R4
    q = q.astype(np.uint8).reshape(N, K)
    return {"q": q, "s": s_st, "z": z_st, "s_bits": s_bits, "z_bits": z_bits,
            "s32": s32, "z32": z32}


# ------------------------------------------------------------- pack/unpack --

def packed_row_bytes(bits: int, K: int) -> int:
    assert (K * bits) % 8 == 0
    return K * bits // 8


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes q[N, K] into the LSB-first contiguous bit stream, uint8 [N, K*b/8].

    Bit j of code k goes to stream position k*b + j; position p is bit p & 7 of
    byte p >> 3 (R8-R10).
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    N, K = q.shape
    if np.any(q >> bits):
        raise ValueError("code out of range for the bit width")
    j = np.arange(bits, dtype=np.uint8)
    stream = ((q[:, :, None] >> j) & 1).astype(np.uint8).reshape(N, K * bits)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of pack: uint8 [N, K*b/8] -> codes uint8 [N, K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, : K * bits]
    stream = stream.reshape(N, K, bits).astype(np.uint16)
    weights = (1 << np.arange(bits, dtype=np.uint16))
    return (stream * weights).sum(axis=2).astype(np.uint8)


def read_code_bitwise(row: bytes, bits: int, k: int) -> int:
    """Pure-Python reader of code k from one row's byte string, one bit at a time.

    For small cases only; it re-derives every bit position from the packing
    rule without any word-level extraction.
    """
    v = 0
    for j in range(bits):
        p = k * bits + j
        if (row[p >> 3] >> (p & 7)) & 1:
            v |= 1 << j
    return v


# ------------------------------------------------------------------ linear --

def dequantize(q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """w[n, k] = s[n, k/group] * q[n, k] + z[n, k/group] in float64 (R1, R11)."""
    q64 = np.asarray(q, dtype=np.float64)
    s64 = np.repeat(np.asarray(s, dtype=np.float64), group, axis=1)
    z64 = np.repeat(np.asarray(z, dtype=np.float64), group, axis=1)
    return s64 * q64 + z64


def linear(x: np.ndarray, q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int,
           bias: Optional[np.ndarray] = None):
    """fp64 reference output and tolerance scale.

    x: [M, K] values of the activations (already rounded to their dtype),
    q: [N, K] codes, s/z: [N, K/group] stored values, bias: [N] or None.
    Returns (y_ref [M, N] float64, A [M, N] float64) with
    y_ref = x . w^T (+ bias) and A = |x| . |w|^T.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = dequantize(q, s, z, group)
    y = x64 @ w64.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    A = np.abs(x64) @ np.abs(w64).T
    return y, A


def tolerance(A: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref| per element: 1e-3 + 2e-3 * sum_k |x_k * w_k|."""
    return 1e-3 + 2e-3 * np.asarray(A, dtype=np.float64)


def linear_rows(x: np.ndarray, q_rows: np.ndarray, s_rows: np.ndarray, z_rows: np.ndarray,
                group: int, bias_rows: Optional[np.ndarray] = None):
    """linear() restricted to a subset of output rows (for sampled parity at full size)."""
    return linear(x, q_rows, s_rows, z_rows, group, bias_rows)


# ----------------------------------------------- dynamic int8 activations --

def quantize_activations_i8(x: np.ndarray):
    """Per-row symmetric int8 quantization of the activations (R30-R32).

    x: [M, K], values of the activations (fp32, or fp16 / bf16 values, which
    are fp32 values).  Returns (xq int8 [M, K], a float32 [M]).
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x32.shape
    xq = np.zeros((M, K), dtype=np.int8)
    a = np.zeros(M, dtype=np.float32)
    for m in range(M):
        row = x32[m]
        if not np.all(np.isfinite(row)):
            a[m] = np.float32(np.nan)                       # R32
            continue
        amax = np.max(np.abs(row))                          # exact
        a[m] = np.float32(amax) / np.float32(127.0)         # fp32 divide
        if a[m] == 0:
            continue                                        # R31
        t = (row / a[m]).astype(np.float32)                 # fp32 divide per element
        xq[m] = np.clip(np.rint(t), -127, 127).astype(np.int8)   # half to even
    return xq, a


def linear_a8(xq: np.ndarray, a: np.ndarray, q: np.ndarray, s: np.ndarray, z: np.ndarray,
              group: int, bias: Optional[np.ndarray] = None):
    """fp64 reference of the linear over int8 activations (R33).

    Returns (y_ref [M, N], A [M, N]) as linear() does, with the activations
    a_m * xq[m, k] (exact in float64).
    """
    xd = np.asarray(a, dtype=np.float64)[:, None] * np.asarray(xq, dtype=np.float64)
    return linear(xd, q, s, z, group, bias)
