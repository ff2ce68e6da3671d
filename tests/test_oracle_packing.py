"""Pins for the oracle's packer / unpacker.

Packing rule: page "metal lowbit kernels: qmv_fast optimization", Summary --
codes stored contiguously across byte boundaries; LSB-first reading (R8).
None of these tests reuses the oracle's own bit-array formulation: they use
hand-derived golden bytes, a Python big-integer formulation of the stream and
a bit-by-bit reader.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing_lsb_first.txt")


def load_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, codes, lsb, msb = [p.strip() for p in line.split("|")]
            rows.append((int(b), [int(c) for c in codes.split()], bytes.fromhex(lsb),
                         None if msb == "-" else bytes.fromhex(msb)))
    return rows


def bigint_pack_row(codes, bits):
    """Independent formulation: the row as one integer, code i at bit offset i*b."""
    v = 0
    for i, c in enumerate(codes):
        v |= int(c) << (i * bits)
    return v.to_bytes(len(codes) * bits // 8, "little")


@pytest.mark.parametrize("row", load_golden(), ids=lambda r: f"b{r[0]}")
def test_golden_vectors(row):
    bits, codes, lsb, msb = row
    got = oracle.pack(np.array([codes], dtype=np.uint8), bits)[0].tobytes()
    assert got == lsb
    if msb is not None:
        assert got != msb
    assert bigint_pack_row(codes, bits) == lsb


@pytest.mark.parametrize("bits", range(1, 8))
@pytest.mark.parametrize("K", [32, 64, 96, 160, 256])
def test_pack_matches_bigint_stream(bits, K):
    rng = np.random.default_rng(100 + bits * 7 + K)
    q = rng.integers(0, 1 << bits, size=(3, K), dtype=np.uint8)
    packed = oracle.pack(q, bits)
    assert packed.shape == (3, K * bits // 8)
    for n in range(3):
        assert packed[n].tobytes() == bigint_pack_row(q[n], bits)


@pytest.mark.parametrize("bits", range(1, 8))
def test_round_trip_and_bitwise_reader(bits):
    rng = np.random.default_rng(7 + bits)
    K = 256
    q = rng.integers(0, 1 << bits, size=(4, K), dtype=np.uint8)
    packed = oracle.pack(q, bits)
    np.testing.assert_array_equal(oracle.unpack(packed, bits, K), q)
    for n in range(4):
        row = packed[n].tobytes()
        assert [oracle.read_code_bitwise(row, bits, k) for k in range(K)] == list(q[n])


@pytest.mark.parametrize("bits", range(1, 8))
def test_size_identity(bits):
    # 8 codes occupy exactly b bytes; 32 codes exactly b 32-bit words.
    q = np.zeros((1, 8), dtype=np.uint8)
    assert oracle.pack(q, bits).shape == (1, bits)
    q = np.zeros((2, 32), dtype=np.uint8)
    assert oracle.pack(q, bits).shape == (2, 4 * bits)


# Codes that straddle a byte boundary inside an 8-code atom, and a 32-bit word
# boundary inside a 32-code atom (closed form: start bit i*b and end bit
# i*b+b-1 fall in different bytes / words).
STRADDLE_BYTE = {3: [2, 5], 5: [1, 3, 4, 6], 6: [1, 2, 5, 6], 7: [1, 2, 3, 4, 5, 6]}
STRADDLE_WORD = {3: [10, 21], 5: [6, 12, 19, 25], 6: [5, 10, 21, 26], 7: [4, 9, 13, 18, 22, 27]}


@pytest.mark.parametrize("bits", [3, 5, 6, 7])
def test_straddling_codes_single_one(bits):
    """A single all-ones code placed at each straddling index sets exactly the
    stream bits [i*b, i*b+b), split across two bytes (or two words)."""
    for idx_list, K, unit in ((STRADDLE_BYTE[bits], 8, 8), (STRADDLE_WORD[bits], 32, 32)):
        for i in idx_list:
            assert (i * bits) // unit != (i * bits + bits - 1) // unit
            q = np.zeros((1, K), dtype=np.uint8)
            q[0, i] = (1 << bits) - 1
            stream = int.from_bytes(oracle.pack(q, bits)[0].tobytes(), "little")
            assert stream == ((1 << bits) - 1) << (i * bits)
    for i in range(8):
        if i not in STRADDLE_BYTE[bits]:
            assert (i * bits) // 8 == (i * bits + bits - 1) // 8


def test_rejects_out_of_range_codes():
    with pytest.raises(ValueError):
        oracle.pack(np.array([[4, 0, 0, 0, 0, 0, 0, 0]], dtype=np.uint8), 2)
