"""The decode kernel's fp16 slot plans (bit_groupwise_weight_amd/csrc/qmv_plan.h),
checked on the CPU against the oracle's packer.

A host harness (tests/plan_harness.cpp) forms each slot word of a run from the
plan tables the way the kernel does (funnel shifts, byte permutes, masks).  For
every width the slots must pair each of a run's 32 codes exactly once, keep
every code below bit 11 of its 16-bit half, and hold exactly the codes the
oracle packed, at the slot's offset o; each half must then read, as an fp16
number, q * 2^(o-24) -- the value the kernel's dot products rely on (the
codes enter as fp16 subnormals, or the first normal binade, whose step is
still 2^-24).  Packing rule: page "metal lowbit kernels: qmv_fast
optimization", Summary (codes stored contiguously across byte boundaries,
LSB first).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "bit_groupwise_weight_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_harness")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "plan_harness.cpp"),
                    "-o", exe], check=True)
    return exe


def codes_for(bits, runs, seed):
    """Random codes plus the edge patterns: all zero, all 2^b - 1, alternating,
    a single set code per run position."""
    rng = np.random.default_rng(seed)
    qmax = (1 << bits) - 1
    rows = [rng.integers(0, qmax + 1, size=32) for _ in range(runs)]
    rows += [np.zeros(32, int), np.full(32, qmax), np.arange(32) % 2 * qmax]
    rows += [np.eye(32, dtype=int)[k] * qmax for k in range(0, 32, 5)]
    return np.array(rows, dtype=np.uint8)


def run_harness(exe, bits, q):
    packed = oracle.pack(q, bits)                    # [runs, 4*b] bytes, LSB-first stream
    words = packed.view("<u4").reshape(-1)           # b words per run
    inp = f"{bits}\n" + " ".join(str(int(w)) for w in words) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [tuple(int(t) for t in line.split()) for line in out.splitlines()]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7])
def test_slot_plan_matches_packed_codes(harness, bits):
    q = codes_for(bits, runs=40, seed=bits)
    rows = run_harness(harness, bits, q)
    nslots = len(rows) // len(q)
    assert nslots * len(q) == len(rows)
    assert nslots == 16                              # two codes per dot2, no dummy halves
    mask = (1 << bits) - 1
    for r, i, klo, khi, o, word in rows:
        assert o >= 0 and o + bits <= 11, (bits, i, o)
        lo, hi = word & 0xffff, word >> 16
        for k, half in ((klo, lo), (khi, hi)):
            want = 0 if k < 0 else int(q[r, k]) << o
            assert half == want, (bits, r, i, k, o, hex(word))
            # the half read as fp16 is q * 2^(o-24), exactly
            val = float(np.array([half], np.uint16).view(np.float16)[0])
            assert val == (0 if k < 0 else float(q[r, k])) * 2.0 ** (o - 24)
        assert (lo & ~(mask << o)) == 0 and (hi & ~(mask << o)) == 0
    # every code of a run sits in exactly one half of one slot
    first = [(klo, khi) for r, i, klo, khi, o, w in rows if r == 0]
    seen = sorted(k for pair in first for k in pair if k >= 0)
    assert seen == list(range(32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7])
def test_slot_plan_reconstructs_the_run_dot(harness, bits):
    """sum over slots of x_lo*lo + x_hi*hi, with each half read as fp16 and
    the slot scaled by 2^(24 - o), is sum_k x_k q_k exactly (integer x here)."""
    q = codes_for(bits, runs=8, seed=100 + bits)
    rows = run_harness(harness, bits, q)
    rng = np.random.default_rng(bits)
    x = rng.integers(-50, 50, size=(len(q), 32))
    tot = np.zeros(len(q))
    for r, i, klo, khi, o, word in rows:
        halves = np.array([word & 0xffff, word >> 16], np.uint16).view(np.float16).astype(np.float64)
        xs = np.array([x[r, klo] if klo >= 0 else 0, x[r, khi] if khi >= 0 else 0], np.float64)
        tot[r] += float(xs @ halves) * 2.0 ** (24 - o)
    want = (x * q.astype(np.int64)).sum(axis=1)
    np.testing.assert_array_equal(tot, want)
