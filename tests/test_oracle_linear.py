"""Pins for the oracle's fp64 dequant-matmul (y = x . dequant(Wq)^T + bias).

Scale/zero indexing [n][k // group]: page "metal lowbit kernels: qmv_fast
optimization", Summary; bias: page "Revamp int4 MPS support in torchao".
The checks use closed forms (one-hot and group-ones inputs), exact integer
arithmetic and exact rational arithmetic -- none of them reuses the oracle's
numpy formulation.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def random_quant(N, K, bits, group, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = (rng.random((N, K // group)) * 0.01 + 1e-3).astype(np.float32)
    z = (rng.standard_normal((N, K // group)) * 0.05).astype(np.float32)
    return q, s, z


@pytest.mark.parametrize("bits,group", [(1, 32), (3, 64), (4, 128), (7, 256)])
def test_one_hot_inputs_pick_single_weights(bits, group):
    N, K = 5, 512
    q, s, z = random_quant(N, K, bits, group, seed=bits)
    x = np.eye(K, dtype=np.float32)            # M = K one-hot rows
    y, A = oracle.linear(x, q, s, z, group)
    for k in range(K):
        g = k // group
        for n in range(N):
            expect = float(s[n, g]) * int(q[n, k]) + float(z[n, g])
            assert y[k, n] == expect
            assert A[k, n] == abs(expect)


@pytest.mark.parametrize("bits,group", [(2, 32), (5, 128), (6, 256)])
def test_group_ones_inputs(bits, group):
    N, K = 4, 1024
    q, s, z = random_quant(N, K, bits, group, seed=bits + 50)
    G = K // group
    x = np.zeros((G, K), dtype=np.float32)
    for g in range(G):
        x[g, g * group:(g + 1) * group] = 1.0
    y, _ = oracle.linear(x, q, s, z, group)
    for g in range(G):
        for n in range(N):
            sq = int(q[n, g * group:(g + 1) * group].astype(np.int64).sum())
            expect = Fraction(float(s[n, g])) * sq + group * Fraction(float(z[n, g]))
            assert abs(Fraction(y[g, n]) - expect) <= abs(expect) * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("bits", range(1, 8))
def test_exact_integer_case(bits):
    """s = 1, z = -2^(b-1), x in {-1, 0, 1}: every partial sum is an integer, so
    the fp64 result must equal the integer matmul exactly."""
    rng = np.random.default_rng(bits + 77)
    M, N, K, group = 3, 7, 1024, 64
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = np.ones((N, K // group), np.float32)
    z = np.full((N, K // group), -(1 << (bits - 1)), np.float32)
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    bias = rng.integers(-5, 6, size=N).astype(np.float32)
    y, _ = oracle.linear(x, q, s, z, group, bias)
    xi = x.astype(np.int64).tolist()
    w = (q.astype(np.int64) - (1 << (bits - 1))).tolist()
    for m in range(M):
        for n in range(N):
            assert y[m, n] == sum(a * b for a, b in zip(xi[m], w[n])) + int(bias[n])


@pytest.mark.parametrize("seed", range(4))
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed + 900)
    M, N, K, group, bits = 3, 4, 256, 32, 3
    q, s, z = random_quant(N, K, bits, group, seed=seed + 1000)
    x = rng.standard_normal((M, K)).astype(np.float16).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float16).astype(np.float32)
    y, A = oracle.linear(x, q, s, z, group, bias)
    for m in range(M):
        for n in range(N):
            acc = Fraction(float(bias[n]))
            absacc = Fraction(0)
            for k in range(K):
                g = k // group
                w = Fraction(float(s[n, g])) * int(q[n, k]) + Fraction(float(z[n, g]))
                acc += Fraction(float(x[m, k])) * w
                absacc += abs(Fraction(float(x[m, k])) * w)
            bound = (K + 2) * Fraction(1, 2 ** 52) * (absacc + abs(Fraction(float(bias[n]))))
            assert abs(Fraction(y[m, n]) - acc) <= bound
            assert abs(Fraction(A[m, n]) - absacc) <= bound


def test_quantize_then_linear_end_to_end_small():
    """Quantize, pack, unpack with the bit reader, then an exact rational matmul."""
    rng = np.random.default_rng(3)
    N, K, group, bits = 3, 64, 32, 5
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((1, K)).astype(np.float16).astype(np.float32)
    out = oracle.quantize(W, bits, group, "f16")
    packed = oracle.pack(out["q"], bits)
    y, _ = oracle.linear(x, out["q"], out["s"], out["z"], group)
    for n in range(N):
        row = packed[n].tobytes()
        acc = Fraction(0)
        for k in range(K):
            code = oracle.read_code_bitwise(row, bits, k)
            w = Fraction(float(out["s"][n, k // group])) * code + Fraction(float(out["z"][n, k // group]))
            acc += Fraction(float(x[0, k])) * w
        assert abs(float(acc) - y[0, n]) <= 1e-12


def test_tolerance_formula():
    A = np.array([0.0, 1.0, 10.0])
    np.testing.assert_allclose(oracle.tolerance(A), [1e-3, 3e-3, 2.1e-2])
