"""Planted mistakes in (copies of) the oracle must be caught by the pins.

Each mutant is a small, plausible error -- a wrong bit order, a transposed
scale index, a dropped zero term, a wrong rounding mode, a swapped sign -- and
each must fail at least one of the closed-form checks the oracle is pinned to.
All on the CPU; the real oracle is never modified.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_packing import bigint_pack_row, load_golden
from tests.test_oracle_quantize import exact_grid_weights


def pack_msb_first(q, bits):
    N, K = q.shape
    j = np.arange(bits)[::-1]
    stream = ((q[:, :, None] >> j) & 1).astype(np.uint8).reshape(N, K * bits)
    return np.packbits(stream, axis=1, bitorder="big")


def pack_code_msb(q, bits):
    # codes in LSB-first byte order but each code's bits reversed
    N, K = q.shape
    j = np.arange(bits)[::-1]
    stream = ((q[:, :, None] >> j) & 1).astype(np.uint8).reshape(N, K * bits)
    return np.packbits(stream, axis=1, bitorder="little")


@pytest.mark.parametrize("mutant", [pack_msb_first, pack_code_msb])
def test_packing_mutants_fail_golden(mutant):
    caught = False
    for bits, codes, lsb, _ in load_golden():
        got = mutant(np.array([codes], np.uint8), bits)[0].tobytes()
        caught |= got != lsb
    assert caught


def linear_transposed_scale(x, q, s, z, group, bias=None):
    # wrong: indexes the scale table as [g][n] by reshaping it
    st = np.ascontiguousarray(s.T).reshape(s.shape)
    return oracle.linear(x, q, st, z, group, bias)


def linear_no_zero(x, q, s, z, group, bias=None):
    return oracle.linear(x, q, s, np.zeros_like(z), group, bias)


def linear_sign_flip(x, q, s, z, group, bias=None):
    return oracle.linear(x, q, s, -z, group, bias)


def linear_group_off_by_one(x, q, s, z, group, bias=None):
    sh = np.roll(s, 1, axis=1)
    return oracle.linear(x, q, sh, z, group, bias)


@pytest.mark.parametrize("mutant", [linear_transposed_scale, linear_no_zero, linear_sign_flip,
                                    linear_group_off_by_one])
def test_linear_mutants_fail_one_hot(mutant):
    rng = np.random.default_rng(1)
    N, K, group = 4, 128, 32
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = (rng.random((N, K // group)) * 0.01 + 1e-3).astype(np.float32)
    z = (rng.standard_normal((N, K // group)) * 0.05).astype(np.float32)
    x = np.eye(K, dtype=np.float32)
    y, _ = mutant(x, q, s, z, group)
    expect = np.array([[float(s[n, k // group]) * int(q[n, k]) + float(z[n, k // group])
                        for n in range(N)] for k in range(K)])
    assert not np.array_equal(y, expect)


def quantize_round_half_up(W, bits, group, dtype):
    out = oracle.quantize(W, bits, group, dtype)
    N, K = W.shape
    s = np.repeat(out["s"], group, axis=1)
    z = np.repeat(out["z"], group, axis=1)
    t = (W - z) / np.where(s == 0, 1, s)
    out["q"] = np.clip(np.floor(t + 0.5), 0, (1 << bits) - 1).astype(np.uint8)
    return out


def quantize_symmetric(W, bits, group, dtype):
    out = oracle.quantize(W, bits, group, dtype)
    N, K = W.shape
    amax = np.abs(W.reshape(N, -1, group)).max(axis=2)
    out["s"] = (2 * amax / ((1 << bits) - 1)).astype(np.float32)
    return out


def test_quantizer_mutants_fail_pins():
    from tests.test_oracle_quantize import test_ties_round_to_even  # noqa: F401
    # round-half-up fails the tie pin
    bits, group = 3, 32
    qmax = 7
    s, z = 2.0 ** -8, -(2.0 ** -3)
    vals = np.array([0, qmax] + [h + 0.5 for h in range(qmax)] * 5)[:group]
    W = (z + s * vals).astype(np.float32)[None, :]
    good = oracle.quantize(W, bits, group, "f32")["q"]
    bad = quantize_round_half_up(W, bits, group, "f32")["q"]
    assert not np.array_equal(good, bad)
    # a symmetric scale fails exact-grid recovery
    W, q, s, z = exact_grid_weights(4, 64)
    assert not np.all(quantize_symmetric(W, 4, 64, "f32")["s"] == np.float32(s))


def test_bigint_formulation_is_not_the_oracle():
    # sanity: the independent formulation really is independent of numpy packbits
    assert bigint_pack_row([1, 2, 3, 4, 5, 6, 7, 0], 3).hex() == "d1581f"


def quantize_codes_from_unrounded(W, bits, group, dtype):
    """Mutant of R6: codes from the fp32 scale and zero before they are rounded
    to the storage dtype (the stored s and z are still returned rounded)."""
    out = oracle.quantize(W, bits, group, dtype)
    N, K = W.shape
    s = np.repeat(out["s32"], group, axis=1).astype(np.float32)
    z = np.repeat(out["z32"], group, axis=1).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((W - z) / np.where(s == 0, np.float32(1), s)).astype(np.float32)
    q = np.clip(np.rint(t), 0, (1 << bits) - 1)
    out["q"] = np.where(s != 0, q, 0).astype(np.uint8)
    return out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_r6_mutant_fails_pins(dtype):
    from tests.test_oracle_quantize import R6_CASES
    for case in R6_CASES:
        W, _, _, codes = case(dtype)
        assert list(quantize_codes_from_unrounded(W, 4, 32, dtype)["q"][0]) != codes
