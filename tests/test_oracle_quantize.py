"""Pins for the oracle's quantizer and storage casts.

Scale/zero layout N x num_groups: page "metal lowbit kernels: qmv_fast
optimization", Summary (first bullet).  Bit widths and groups: page "Add
torchao mps ops".  Quantizer formula (asymmetric min/max, R2-R7, R22) is a
reading; the pins below are closed forms that any correct implementation of it
must reproduce.
"""
import numpy as np
import pytest
import torch

import oracle

DTYPES = ["f32", "f16", "bf16"]


# ----------------------------------------------------------- storage casts --

def test_f16_cast_textbook_values():
    # binary16: 1 + 2^-11 is a tie -> 1.0 (even); 1 + 3*2^-11 -> 1 + 2^-9;
    # 65519.996 -> 65504, 65520 -> inf; 2^-24 is the smallest subnormal, 2^-25 ties to 0.
    vals = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65519.0, 65520.0, 2.0 ** -24,
                     2.0 ** -25, 3 * 2.0 ** -25, -0.0], dtype=np.float32)
    got, bits = oracle.round_to_storage(vals, "f16")
    exp = np.array([1.0, 1 + 2.0 ** -9, 65504.0, np.inf, 2.0 ** -24, 0.0, 2.0 ** -23, -0.0])
    np.testing.assert_array_equal(got, exp.astype(np.float32))
    assert bits[-1] == 0x8000 and bits[0] == 0x3C00


def test_bf16_cast_textbook_values():
    # bf16 keeps 8 significant bits: 1 + 2^-8 ties to 1.0; 1 + 3*2^-8 -> 1 + 2^-6;
    # largest finite 3.3895e38 (0x7F7F); values past the rounding boundary go to inf.
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,
                     3.3895313892515355e38, np.float32(3.4028235e38), -2.0], dtype=np.float32)
    _, bits = oracle.round_to_storage(vals, "bf16")
    assert list(bits) == [0x3F80, 0x3F82, 0x3F81, 0x7F7F, 0x7F80, 0xC000]


def test_bf16_cast_matches_torch():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    a = u.view(np.float32)
    a = a[np.isfinite(a)]
    a = np.concatenate([a, rng.standard_normal(100000).astype(np.float32) * 0.02,
                        np.array([0.0, -0.0, 1e-40, -1e-40], dtype=np.float32)])
    _, bits = oracle.round_to_storage(a, "bf16")
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_f16_cast_matches_torch():
    rng = np.random.default_rng(6)
    a = (rng.standard_normal(200000) * rng.choice([1e-6, 1e-3, 1.0, 1e3, 6e4], 200000)).astype(np.float32)
    _, bits = oracle.round_to_storage(a, "f16")
    ref = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


# --------------------------------------------------------------- quantizer --

def exact_grid_weights(bits, group, N=3, G=4, seed=0):
    """W = z + s*q with s = 2^-8, z = -2^-3, every group containing codes 0 and
    2^b-1; exact in fp32, fp16 and bf16."""
    rng = np.random.default_rng(seed)
    qmax = (1 << bits) - 1
    q = rng.integers(0, qmax + 1, size=(N, G, group))
    q[:, :, 0] = 0
    q[:, :, -1] = qmax
    rng.permuted(q, axis=2, out=q)
    s, z = 2.0 ** -8, -(2.0 ** -3)
    W = (z + s * q).astype(np.float32).reshape(N, G * group)
    return W, q.reshape(N, G * group).astype(np.uint8), s, z


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", range(1, 8))
def test_exact_grid_recovery(bits, group, dtype):
    W, q, s, z = exact_grid_weights(bits, group, seed=bits * 10 + group)
    out = oracle.quantize(W, bits, group, dtype)
    np.testing.assert_array_equal(out["q"], q)
    assert np.all(out["s"] == np.float32(s)) and np.all(out["z"] == np.float32(z))
    assert out["s"].shape == (W.shape[0], W.shape[1] // group)   # N x num_groups


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bits", [2, 3, 4, 7])
def test_ties_round_to_even(bits, dtype):
    group = 32
    qmax = (1 << bits) - 1
    s, z = 2.0 ** -8, -(2.0 ** -3)
    vals = np.zeros(group)
    vals[0], vals[1] = 0, qmax
    halves = [h + 0.5 for h in range(qmax)]
    for i in range(2, group):
        vals[i] = halves[(i - 2) % len(halves)]
    W = (z + s * vals).astype(np.float32)[None, :]
    out = oracle.quantize(W, bits, group, dtype)
    expect = [0, qmax] + [int(h) + (int(h) % 2) for h in (vals[2:] - 0.5)]
    assert list(out["q"][0]) == expect


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("c", [0.0, -0.0, 0.3, -1.7, 1e-3])
def test_constant_group(dtype, c):
    W = np.full((2, 64), c, dtype=np.float32)
    out = oracle.quantize(W, 4, 64, dtype)
    assert np.all(out["q"] == 0)
    assert np.all(out["s"] == 0) and np.all(out["s_bits"] == 0)
    zc, zbits = oracle.round_to_storage(np.array([abs(c) if c == 0 else c], np.float32), dtype)
    assert np.all(out["z_bits"] == zbits[0])   # a zero minimum is stored as +0 (R22)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bits", range(1, 8))
def test_invariants_and_reconstruction_bound(bits, dtype):
    rng = np.random.default_rng(bits + 31)
    N, K, group = 16, 512, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    out = oracle.quantize(W, bits, group, dtype)
    q, s, z = out["q"], out["s"].astype(np.float64), out["z"].astype(np.float64)
    qmax = (1 << bits) - 1
    assert q.min() >= 0 and q.max() <= qmax
    wg = W.reshape(N, -1, group).astype(np.float64)
    what = oracle.dequantize(q, out["s"], out["z"], group).reshape(N, -1, group)
    mn = wg.min(axis=2)
    s32 = out["s32"].astype(np.float64)
    bound = (0.5 * s + qmax * np.abs(s32 - s) + np.abs(mn - z))[:, :, None] * (1 + 1e-5) + 1e-12
    assert np.all(np.abs(wg - what) <= bound)
    if dtype == "f32":
        qg = q.reshape(N, -1, group)
        am, aM = wg.argmin(axis=2), wg.argmax(axis=2)
        assert np.all(np.take_along_axis(qg, am[:, :, None], 2) == 0)
        assert np.all(np.take_along_axis(qg, aM[:, :, None], 2) == qmax)


def frac_to_f32(fr):
    """Round an exact rational to the nearest fp32 (ties to even), without
    going through float64 first."""
    from fractions import Fraction
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    errs = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(errs)
    tied = [c for c, e in zip(cands, errs) if e == best]
    if len(tied) > 1:
        tied = [c for c in tied if int(np.array(c, np.float32).view(np.uint32)) % 2 == 0]
    return tied[0]


def test_scale_formula_single_group():
    # s = (max - min) / (2^b - 1) as two single roundings: compare with exact
    # rational arithmetic rounded to fp32 once per operation.
    from fractions import Fraction
    for seed in range(20):
        rng = np.random.default_rng(seed)
        W = (rng.standard_normal((1, 64)) * 0.05).astype(np.float32)
        for bits in (3, 5, 7):
            out = oracle.quantize(W, bits, 64, "f32")
            diff = frac_to_f32(Fraction(float(W.max())) - Fraction(float(W.min())))
            s = frac_to_f32(Fraction(float(diff)) / ((1 << bits) - 1))
            assert out["s"][0, 0] == s
            assert out["z"][0, 0] == W.min()
            # codes: t = (w - z) / s, each op rounded once, then half-to-even
            for k in range(64):
                num = frac_to_f32(Fraction(float(W[0, k])) - Fraction(float(W.min())))
                t = frac_to_f32(Fraction(float(num)) / Fraction(float(s)))
                assert out["q"][0, k] == min(max(int(np.rint(t)), 0), (1 << bits) - 1)


def test_rejects_nonfinite_and_range():
    W = np.zeros((1, 32), np.float32)
    W[0, 5] = np.nan
    with pytest.raises(oracle.NonFiniteInput):
        oracle.quantize(W, 4, 32, "f16")
    W = np.zeros((1, 32), np.float32)
    W[0, 1] = 1e6          # scale 1e6/15 fits fp16? no: z=0 ok, s=66666 > 65504
    with pytest.raises(oracle.RangeError):
        oracle.quantize(W, 4, 32, "f16")
    oracle.quantize(W, 4, 32, "f32")   # fine in fp32
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((1, 48), np.float32), 4, 32, "f16")
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((1, 64), np.float32), 8, 32, "f16")


# ------------------------------------------------- R6: order of rounding --
# Codes are computed from the STORED (rounded) scale and zero, not from the
# fp32 values before rounding.  Each case below is derived by hand so that the
# two rules give different codes; the page "metal lowbit kernels: qmv_fast
# optimization" (Summary) has the kernels consume scales and zeros exactly as
# the quantize function stores them, so the codes must be a function of those
# stored values.

def _r6_scale_case(dtype):
    """Group of 32 at 4 bits: min 0, max 1, and one weight w.

    s32 = fp32(1/15).  Stored: fp16 1/15 -> 1092 * 2^-14 = 0.066650390625
    (bits 0x2C44, below 1/15); bf16 1/15 -> 137 * 2^-11 = 0.06689453125 (bits
    0x3D89, above 1/15).  z = 0 is exact in every dtype.
      fp16, w = 0.9665: w / s_st = 14.501 -> 15, while 15 * w = 14.4975 -> 14.
      bf16, w = 0.968:  w / s_st = 14.471 -> 14, while 15 * w = 14.52 -> 15.
    """
    w, s_bits, code_w = {"f16": (0.9665, 0x2C44, 15), "bf16": (0.968, 0x3D89, 14)}[dtype]
    W = np.zeros((1, 32), np.float32)
    W[0, 1], W[0, 2] = 1.0, w
    return W, s_bits, 0x0000, [0, 15, code_w] + [0] * 29


def _r6_zero_case(dtype):
    """Group of 32 at 4 bits: min = fp32(-0.1) (bits 0xBDCCCCCD), max = min +
    15 * 2^-6 (fp32 bits 0x3E09999A), so s = 2^-6 exactly in every dtype.
    Stored zero: fp16 -0.1 -> -0.0999755859375 (0xAE66, 2.44e-5 above);
    bf16 -0.1 -> -0.10009765625 (0xBDCD, 9.77e-5 below).
      fp16, w bits 0x3C8CED90: (w - z32) / s = 7.5010 -> 8, (w - z_st) / s = 7.4994 -> 7.
      bf16, w bits 0x3C8C6A80: (w - z32) / s = 7.4970 -> 7, (w - z_st) / s = 7.5033 -> 8.
    """
    wbits, z_bits, s_bits, code_w = {"f16": (0x3C8CED90, 0xAE66, 0x2400, 7),
                                      "bf16": (0x3C8C6A80, 0xBDCD, 0x3C80, 8)}[dtype]
    W = np.zeros((1, 32), np.float32)
    W[0, 0] = np.float32(-0.1)
    W[0, 1] = np.array([0x3E09999A], np.uint32).view(np.float32)[0]
    W[0, 2] = np.array([wbits], np.uint32).view(np.float32)[0]
    W[0, 3:] = W[0, 0]
    return W, s_bits, z_bits, [0, 15, code_w] + [0] * 29


R6_CASES = [_r6_scale_case, _r6_zero_case]


@pytest.mark.parametrize("case", R6_CASES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_r6_codes_from_stored_scale_and_zero(case, dtype):
    W, s_bits, z_bits, codes = case(dtype)
    out = oracle.quantize(W, 4, 32, dtype)
    assert int(out["s_bits"][0, 0]) == s_bits
    assert int(out["z_bits"][0, 0]) == z_bits
    assert list(out["q"][0]) == codes
