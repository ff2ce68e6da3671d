"""Pins of the oracle's dynamic int8 activation quantizer and its linear.

The activation-quantized variant is the "-qmode 8da4w -G 32" export mode of
"[MPS] Add support for Int4 groupwise quantization" (8-bit dynamic
activations, 4-bit weights, groups of 32).  The page names the mode only; the
oracle's readings fix the arithmetic: one fp32 scale per row,
a = max|x| / 127, codes rint_half_even(x / a) clamped to [-127, 127], both
divides in fp32; a zero row has codes 0; a non-finite row has a = NaN and
codes 0.  These tests check the oracle against things that do not reuse its
formula: hand-derived rows, an exact-rational re-derivation of every rounding
step, exact grids, invariants of a symmetric quantizer, and brute-force
integer sums for the linear.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def nearest_f32(r: Fraction) -> Fraction:
    """The fp32 value nearest to r (ties to an even significand), normal range."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    r = abs(r)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    assert -126 <= e <= 127, "test values stay in the normal range"
    ulp = Fraction(2) ** (e - 23)
    n = r / ulp                      # in [2^23, 2^24)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_half_even(r: Fraction) -> int:
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def exact_quantize_row(row):
    """The reading's steps on exact rationals: fp32 roundings made explicit."""
    vals = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in vals)
    if amax == 0:
        return [0] * len(vals), Fraction(0)
    a = nearest_f32(amax / 127)
    codes = []
    for v in vals:
        t = nearest_f32(v / a) if v != 0 else Fraction(0)
        codes.append(max(-127, min(127, round_half_even(t))))
    return codes, a


# ------------------------------------------------------------ quantizer --

def test_hand_derived_row_with_unit_scale():
    # max |x| = 127, so a = 1 exactly and every code is x rounded half to even
    x = np.array([[1.0, -2.0, 0.5, 127.0, 2.5, 3.5, -2.5, -0.5, 1.5, -126.5, 0.0, 64.25]],
                 np.float32)
    xq, a = oracle.quantize_activations_i8(x)
    assert a[0] == np.float32(1.0)
    assert xq[0].tolist() == [1, -2, 0, 127, 2, 4, -2, 0, 2, -126, 0, 64]
    assert xq.dtype == np.int8


@pytest.mark.parametrize("c", [3, 255])
def test_ties_at_a_scale_that_is_not_a_power_of_two(c):
    # max |x| = 127 c 2^-10 gives a = c 2^-10 exactly (c odd); x = (2k + 1) c 2^-11
    # is exactly k + 1/2 scales: a tie, which goes to the even code.  (The
    # reciprocal 2^10 / c is not an fp32 value; at c = 255 its rounding moves
    # about half of these ties, so x * (1/a) in place of x / a fails here.)
    ks = list(range(-127, 127))
    row = [127.0 * c * 2.0 ** -10] + [(2 * k + 1) * c * 2.0 ** -11 for k in ks]
    xq, a = oracle.quantize_activations_i8(np.array([row], np.float32))
    assert a[0] == np.float32(c * 2.0 ** -10)
    expect = [127] + [k if k % 2 == 0 else k + 1 for k in ks]
    assert xq[0].tolist() == expect


def test_unit_row_scale_is_the_nearest_fp32_to_one_127th():
    x = np.array([[0.25, -1.0, 0.5, 0.75, -0.125]], np.float32)
    xq, a = oracle.quantize_activations_i8(x)
    assert Fraction(float(a[0])) == nearest_f32(Fraction(1, 127))
    assert xq[0].tolist() == exact_quantize_row(x[0])[0]
    assert xq[0, 1] == -127


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_exact_rational_rederivation(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((6, 48)).astype(np.float32)
    x[1] *= np.float32(1e-3)
    x[2, 5] = np.float32(40.0)                  # an outlier sets the scale
    x[3] = np.round(x[3] * 8) / 8               # values on a coarse grid
    x[4, :] = np.float32(-3.0)                  # a constant row
    xq, a = oracle.quantize_activations_i8(x)
    for m in range(x.shape[0]):
        codes, a_exact = exact_quantize_row(x[m])
        assert Fraction(float(a[m])) == a_exact
        assert xq[m].tolist() == codes


@pytest.mark.parametrize("shift", [-3, 0, 2])
def test_exact_grid_recovery(shift):
    # a power-of-two scale: rows of k * 2^shift with max |k| = 127 give
    # a = 2^shift and codes k exactly
    rng = np.random.default_rng(7)
    k = rng.integers(-127, 128, size=(5, 64))
    k[:, 0] = 127 * np.where(rng.random(5) < 0.5, -1, 1)
    x = (k * 2.0 ** shift).astype(np.float32)
    xq, a = oracle.quantize_activations_i8(x)
    assert np.all(a == np.float32(2.0 ** shift))
    np.testing.assert_array_equal(xq, k.astype(np.int8))


def test_invariants_of_a_symmetric_quantizer():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 20
    xq, a = oracle.quantize_activations_i8(x)
    # the element of largest magnitude takes the extreme code of its sign
    idx = np.argmax(np.abs(x), axis=1)
    rows = np.arange(x.shape[0])
    assert np.all(xq[rows, idx] == np.where(x[rows, idx] > 0, 127, -127))
    assert np.all(np.abs(xq.astype(np.int32)) <= 127)
    # reconstruction within half a step (plus the divide's rounding)
    err = np.abs(x.astype(np.float64) - a[:, None].astype(np.float64) * xq)
    assert np.all(err <= a[:, None] * (0.5 + 2.0 ** -16))
    # negation: same scale, negated codes
    xq_n, a_n = oracle.quantize_activations_i8(-x)
    np.testing.assert_array_equal(a_n, a)
    np.testing.assert_array_equal(xq_n, -xq)
    # a power-of-two scaling of a row scales a exactly and keeps the codes
    for j in (-5, 3):
        xq_s, a_s = oracle.quantize_activations_i8((x * np.float32(2.0 ** j)).astype(np.float32))
        np.testing.assert_array_equal(xq_s, xq)
        np.testing.assert_array_equal(a_s, (a * np.float32(2.0 ** j)).astype(np.float32))


def test_zero_and_nonfinite_rows():
    x = np.ones((5, 32), np.float32)
    x[0] = 0.0
    x[1, 3] = np.nan
    x[2, 0] = np.inf
    x[3, 31] = -np.inf
    x[4, 7] = -0.0
    xq, a = oracle.quantize_activations_i8(x)
    assert a[0] == 0 and not np.any(xq[0])
    for m in (1, 2, 3):
        assert np.isnan(a[m]) and not np.any(xq[m])
    assert a[4] == np.float32(1.0) / np.float32(127.0)
    assert xq[4, 7] == 0 and np.all(np.delete(xq[4], 7) == 127)


# --------------------------------------------------------------- linear --

def test_linear_a8_brute_force_integer_sums():
    # exact rational arithmetic: dyadic a, s, z and integer codes
    rng = np.random.default_rng(3)
    M, N, K, group, bits = 3, 5, 64, 32, 4
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a = np.array([2.0 ** -3, 2.0 ** -7, 0.5], np.float32)
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    s = (rng.integers(1, 9, size=(N, K // group)) * 2.0 ** -6).astype(np.float32)
    z = (rng.integers(-40, 40, size=(N, K // group)) * 2.0 ** -5).astype(np.float32)
    bias = (rng.integers(-8, 8, size=N) * 0.25).astype(np.float32)
    y, A = oracle.linear_a8(xq, a, q, s, z, group, bias)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            absum = Fraction(0)
            for g in range(K // group):
                P = sum(int(xq[m, k]) * int(q[n, k]) for k in range(g * group, (g + 1) * group))
                X = sum(int(xq[m, k]) for k in range(g * group, (g + 1) * group))
                tot += Fraction(float(s[n, g])) * P + Fraction(float(z[n, g])) * X
                for k in range(g * group, (g + 1) * group):
                    w = Fraction(float(s[n, g])) * int(q[n, k]) + Fraction(float(z[n, g]))
                    absum += abs(int(xq[m, k]) * w)
            expect = Fraction(float(a[m])) * tot + Fraction(float(bias[n]))
            assert Fraction(float(y[m, n])) == expect
            assert Fraction(float(A[m, n])) == Fraction(float(a[m])) * absum


def test_linear_a8_one_hot_and_nan_row():
    K, group = 64, 64
    xq = np.zeros((2, K), np.int8)
    xq[0, 17] = -5
    a = np.array([0.25, np.nan], np.float32)
    q = np.zeros((2, K), np.uint8)
    q[0, 17] = 9
    q[1, 17] = 3
    s = np.array([[0.5], [2.0]], np.float32)
    z = np.array([[-1.0], [0.125]], np.float32)
    bias = np.array([1.0, -2.0], np.float32)
    y, _ = oracle.linear_a8(xq, a, q, s, z, group, bias)
    # row 0: 0.25 * (-5) * (s*q + z) + bias
    assert y[0, 0] == 0.25 * -5 * (0.5 * 9 - 1.0) + 1.0
    assert y[0, 1] == 0.25 * -5 * (2.0 * 3 + 0.125) - 2.0
    assert np.all(np.isnan(y[1]))


# ---------------------------------------------------------------- mutants --

def q_round_half_away(x):
    x32 = np.asarray(x, np.float32)
    a = (np.max(np.abs(x32), axis=1) / np.float32(127)).astype(np.float32)
    t = (x32 / a[:, None]).astype(np.float32)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8), a


def q_scale_128(x):
    x32 = np.asarray(x, np.float32)
    a = (np.max(np.abs(x32), axis=1) / np.float32(128)).astype(np.float32)
    t = (x32 / a[:, None]).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8), a


def q_signed_max(x):
    x32 = np.asarray(x, np.float32)
    a = (np.max(x32, axis=1) / np.float32(127)).astype(np.float32)
    t = (x32 / a[:, None]).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8), a


def q_reciprocal(x):
    x32 = np.asarray(x, np.float32)
    a = (np.max(np.abs(x32), axis=1) / np.float32(127)).astype(np.float32)
    t = (x32 * (np.float32(1) / a)[:, None]).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8), a


@pytest.mark.parametrize("mutant", [q_round_half_away, q_scale_128, q_signed_max, q_reciprocal])
def test_quantizer_mutants_fail_pins(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "quantize_activations_i8", mutant)
    failed = 0
    for pin in (test_hand_derived_row_with_unit_scale,
                lambda: test_ties_at_a_scale_that_is_not_a_power_of_two(255),
                test_unit_row_scale_is_the_nearest_fp32_to_one_127th):
        try:
            pin()
        except AssertionError:
            failed += 1
    for seed in (0, 1):
        try:
            test_exact_rational_rederivation(seed)
        except AssertionError:
            failed += 1
    try:
        test_invariants_of_a_symmetric_quantizer()
    except AssertionError:
        failed += 1
    assert failed > 0


_real_linear_a8 = oracle.linear_a8


def linear_a8_bias_scaled(xq, a, q, s, z, group, bias=None):
    y, A = _real_linear_a8(xq, a, q, s, z, group, None)
    return y + np.asarray(a, np.float64)[:, None] * np.asarray(bias, np.float64)[None, :], A


def linear_a8_no_act_scale(xq, a, q, s, z, group, bias=None):
    return _real_linear_a8(xq, np.ones_like(a), q, s, z, group, bias)


@pytest.mark.parametrize("mutant", [linear_a8_bias_scaled, linear_a8_no_act_scale])
def test_linear_mutants_fail_pins(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "linear_a8", mutant)
    with pytest.raises(AssertionError):
        test_linear_a8_brute_force_integer_sums()
