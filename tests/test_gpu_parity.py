"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: codes, packed bytes, scales and zeros.  Outputs: within
1e-3 + 2e-3 * sum_k |x_k w_k| per element of the fp64 reference; bit-exact when
every intermediate is an exact integer.  Small shapes are compared in full
(several tiles plus ragged tails); the workloads' full shapes are compared on
sampled rows that the oracle computes one by one.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd.workloads import Case, all_cases, make_bias, make_x
from tests.gpu_helpers import (DEV, TORCH_ACT, act_bits, bias_values, check_close, upload_quant,
                               weight_for, x_values)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module", autouse=True)
def _lib(lowbit_lib):
    return lowbit_lib


def gpu_quantize(W: torch.Tensor, bits, group, act, want_codes=True):
    return lb.lowbit_quantize_pack(W.to(DEV), bits, group, TORCH_ACT[act], want_codes=want_codes)


def assert_quant_equal(ref, packed, s, z, codes, bits, rows=None):
    sel = slice(None) if rows is None else rows
    if codes is not None:
        np.testing.assert_array_equal(codes.cpu().numpy()[sel], ref["q"])
    np.testing.assert_array_equal(packed.cpu().numpy()[sel], oracle.pack(ref["q"], bits))
    np.testing.assert_array_equal(act_bits(s)[sel], ref["s_bits"])
    np.testing.assert_array_equal(act_bits(z)[sel], ref["z_bits"])


# ------------------------------------------------------------- quantizer --

SMALL_K = {32: [32, 96, 352], 64: [64, 320], 128: [128, 384], 256: [256, 768]}


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", range(1, 8))
def test_quantize_small(bits, group, act):
    for K in SMALL_K[group]:
        case = Case("q", 1, K, 67, bits, group, act, seed=bits * 1000 + K)
        W = weight_for(case)
        ref = oracle.quantize(W.numpy(), bits, group, act)
        packed, s, z, codes = gpu_quantize(W, bits, group, act)
        torch.cuda.synchronize()
        assert_quant_equal(ref, packed, s, z, codes, bits)


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
def test_quantize_edge_values(act):
    """Constant groups, signed zeros, exact grids, ties, subnormal weights and
    scales, and the order-of-rounding cases, inside real rows."""
    rng = np.random.default_rng(11)
    bits, group, K, N = 4, 32, 256, 11
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :32] = 0.0
    W[0, 32:64] = -0.0
    W[1, :64] = 0.37
    W[2, 64:96] = np.where(np.arange(32) % 2 == 0, -0.0, 0.0)
    W[3, :32] = (-(2.0 ** -3) + 2.0 ** -8 * (np.arange(32) % 16)).astype(np.float32)
    W[3, 32:64] = (-(2.0 ** -3) + 2.0 ** -8 * ((np.arange(32) % 15) + 0.5)).astype(np.float32)
    W[3, 32], W[3, 33] = -(2.0 ** -3), -(2.0 ** -3) + 15 * 2.0 ** -8
    W[4, :] = 1e-30
    # fp32-subnormal weights (below 2^-126), alone and mixed with normal ones
    W[5, :32] = (np.arange(32) * 3e-42).astype(np.float32)
    W[5, 32:64] = (rng.standard_normal(32) * 1e-38).astype(np.float32)
    # scales that are fp16 subnormals (below 2^-14): max - min = 0.7 * 2^-14
    W[6, :32] = (np.linspace(0.0, 0.7 * 2.0 ** -14, 32) + 0.25).astype(np.float32)
    W[6, 32:64] = (rng.random(32) * 2.0 ** -17).astype(np.float32)
    W[6, 32] = 0.0
    # the hand-derived order-of-rounding groups of the oracle's R6 pins
    from tests.test_oracle_quantize import R6_CASES
    for i, case in enumerate(R6_CASES):
        Wc, _, _, _ = case("f16" if act == "f32" else act)
        W[7 + i, :32] = Wc[0]
    Wt = torch.from_numpy(W)
    ref = oracle.quantize(W, bits, group, act)
    packed, s, z, codes = gpu_quantize(Wt, bits, group, act)
    torch.cuda.synchronize()
    assert_quant_equal(ref, packed, s, z, codes, bits)


@pytest.mark.parametrize("w_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("sz", ["f32", "f16", "bf16"])
def test_quantize_half_precision_weights(w_dtype, sz):
    """fp16 / bf16 weights are taken exactly as fp32 (every such value is an
    fp32 value): bit-exact against the oracle on the upcast weights, for
    every storage dtype of the scales and zeros."""
    rng = np.random.default_rng(17)
    for bits, group, N, K in [(4, 64, 37, 512), (3, 32, 9, 96), (7, 256, 20, 768)]:
        W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        Wh = W.to(TORCH_ACT[w_dtype])
        ref = oracle.quantize(Wh.float().numpy(), bits, group, sz)
        packed, s, z, codes = lb.lowbit_quantize_pack(Wh.to(DEV), bits, group, TORCH_ACT[sz],
                                                      want_codes=True)
        torch.cuda.synchronize()
        assert_quant_equal(ref, packed, s, z, codes, bits)


def test_quantize_errors():
    W = torch.zeros(4, 64)
    W[2, 5] = float("nan")
    with pytest.raises(lb.LowbitError) as e:
        gpu_quantize(W, 4, 32, "f16")
    assert e.value.status_name == "LOWBIT_ERR_NONFINITE"
    W = torch.zeros(4, 64)
    W[1, 3] = float("inf")
    with pytest.raises(lb.LowbitError):
        gpu_quantize(W, 4, 32, "bf16")
    W = torch.zeros(4, 64)
    W[0, 1] = 1e6
    with pytest.raises(lb.LowbitError) as e:
        gpu_quantize(W, 4, 32, "f16")
    assert e.value.status_name == "LOWBIT_ERR_RANGE"
    # the status word is cleared between calls: a good call after a bad one succeeds
    gpu_quantize(torch.zeros(4, 64), 4, 32, "f16")


def test_quantize_concurrent_status():
    """Calls from two threads on one device, one with a NaN weight and one
    clean, each report their own status (the per-device status word is held
    for the whole call), over many rounds on separate streams."""
    import threading
    bad = torch.zeros(64, 256)
    bad[7, 100] = float("nan")
    good = torch.randn(64, 256) * 0.02
    errors = []

    def worker(W, want):
        stream = torch.cuda.Stream(device=DEV)
        try:
            with torch.cuda.stream(stream):
                for _ in range(25):
                    try:
                        gpu_quantize(W, 4, 32, "f16", want_codes=False)
                        got = "LOWBIT_OK"
                    except lb.LowbitError as e:
                        got = e.status_name
                    if got != want:
                        errors.append((want, got))
        except Exception as e:   # reported below, not swallowed
            errors.append(("exception", repr(e)))

    threads = [threading.Thread(target=worker, args=(bad, "LOWBIT_ERR_NONFINITE")),
               threading.Thread(target=worker, args=(good, "LOWBIT_OK"))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


# ---------------------------------------------------------------- linear --

def run_small_linear(M, N, K, bits, group, act, bias, path, seed):
    case = Case("l", M, K, N, bits, group, act, bias=bias, seed=seed)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, bits, group, act)
    x = make_x(case)
    b = make_bias(case)
    y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], group, bias_values(b))
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
    y = lb.lowbit_linear(x.to(DEV), packed, s, z, None if b is None else b.to(DEV), bits, group,
                         path=path)
    torch.cuda.synchronize()
    return check_close(y, y_ref, A, f"M={M} N={N} K={K} b={bits} g={group} {act} path={path}")


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmv_small(bits, act):
    for (M, N, K, group, bias) in [(1, 200, 384, 64, False), (1, 67, 352, 32, True),
                                   (2, 33, 768, 256, True), (3, 130, 8448, 128, False),
                                   (5, 17, 160, 32, True), (15, 9, 640, 64, False),
                                   (1, 1, 32, 32, True)]:
        run_small_linear(M, N, K, bits, group, act, bias, lb.PATH_QMV, seed=bits + M + K)


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmv_long_rows(bits, act):
    """Rows longer than 64 lanes of four 32-code runs (K > 8192), which the
    decode kernel takes in several rounds: K just past 8192 and 14336 (a
    ragged second round), 16384 (two exact rounds), just past 16384 (a third
    round of one run per lane group); one and two activation rows."""
    for (M, N, K, group, bias) in [(1, 37, 8224, 32, True), (1, 70, 14336, 64, False),
                                   (1, 33, 16384, 256, True), (1, 20, 16416, 32, False),
                                   (2, 24, 14336, 128, True)]:
        run_small_linear(M, N, K, bits, group, act, bias, lb.PATH_QMV, seed=bits + M + K)


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmm_small(bits, act):
    # fp16 at M <= 16 runs the small-M kernel; with qmm_small_m=1 the tiled
    # kernel takes those rows too
    for small_m in (0, 1):
        if small_m and act != "f16":
            continue
        with lb.tuning(qmm_small_m=small_m):
            for (M, N, K, group, bias) in [(16, 64, 256, 64, False), (17, 130, 352, 32, True),
                                           (64, 70, 768, 256, True), (100, 200, 384, 128, False),
                                           (1, 5, 64, 32, True), (130, 64, 1024, 64, True)]:
                run_small_linear(M, N, K, bits, group, act, bias, lb.PATH_QMM, seed=bits + M + K)


@pytest.mark.parametrize("nt,waves", [("1", "0"), ("1", "4"), ("2", "8"), ("1", "16")])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmm_small_m_kernel(bits, nt, waves):
    """The small-M fp16 kernel: every M from 1 to 16, columns past N, a last
    K step of 32, a single 32-long run, K ranges that leave waves without
    steps or with an odd number of two-step chunks, every group size."""
    with lb.tuning(qmm_small_m=16, qmm_nt=int(nt), qmm_waves=int(waves)):
        for (M, N, K, group, bias) in [(1, 40, 416, 32, True), (2, 300, 1024, 64, False),
                                       (3, 17, 32, 32, True), (4, 130, 2176, 128, True),
                                       (5, 64, 768, 256, False), (8, 257, 4096, 128, True),
                                       (11, 96, 1280, 256, True), (13, 33, 640, 32, False),
                                       (16, 200, 3328, 64, True), (16, 48, 14336, 128, False)]:
            run_small_linear(M, N, K, bits, group, "f16", bias, lb.PATH_QMM, seed=bits + 7 * M + N)


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmv_register_variants(bits, act):
    """The decode-kernel variants for one activation row (the default, the
    register-lean one, and the lean ones with two or one rows per lane group,
    chosen by blocks and waves per CU) on ragged shapes: each matches the oracle, and all
    agree bit for bit (they differ in register use and in which rows share a
    lane group, not in the arithmetic of a row)."""
    for (N, K, group, bias) in [(200, 384, 64, True), (67, 352, 32, False), (130, 1024, 256, True)]:
        case = Case("v", 1, K, N, bits, group, act, bias=bias, seed=bits * 7 + N)
        W = weight_for(case).numpy()
        ref = oracle.quantize(W, bits, group, act)
        x, b = make_x(case), make_bias(case)
        y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], group, bias_values(b))
        packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
        outs = []
        for variant in (0, 1, 2, 3):
            with lb.tuning(qmv_variant=variant + 1):
                y = lb.lowbit_linear(x.to(DEV), packed, s, z, None if b is None else b.to(DEV), bits,
                                     group, path=lb.PATH_QMV)
            torch.cuda.synchronize()
            check_close(y, y_ref, A, f"variant={variant} N={N} K={K} b={bits} g={group} {act}")
            outs.append(y)
        for y in outs[1:]:
            assert torch.equal(outs[0], y), f"variants differ: N={N} K={K} b={bits} {act}"


@pytest.mark.parametrize("waves,kgroups,nt", [("4", "1", "2"), ("8", "1", "2"), ("4", "2", "2"),
                                               ("4", "2", "1")])
@pytest.mark.parametrize("bits", [1, 3, 4, 5, 7])
def test_qmm_block_variants(bits, waves, kgroups, nt):
    """Every MFMA block shape (4 waves x 128 columns; 8 waves x 256 columns;
    4 column waves x 2 K groups over 128 or 64 columns) on ragged shapes: rows
    past M, columns past N, a last K step of 32, an odd step count (17) so
    that one K group gets a step past the block's range.  8-wave instances
    exist up to 5 bits and K-group instances up to 4; above, the 4-wave kernel
    runs."""
    with lb.tuning(qmm_waves=int(waves), qmm_kgroups=int(kgroups), qmm_nt=int(nt)):
        for (M, N, K, group, bias) in [(128, 300, 416, 32, True), (100, 520, 1024, 64, False),
                                       (77, 257, 2080, 32, True), (128, 130, 2176, 128, False)]:
            run_small_linear(M, N, K, bits, group, "f16", bias, lb.PATH_QMM, seed=bits + N)


@pytest.mark.parametrize("rgroups,nt", [("1", "2"), ("2", "2"), ("1", "1")])
@pytest.mark.parametrize("bits", [1, 3, 4, 6, 7])
def test_qmm_bf16_block_variants(bits, rgroups, nt):
    """bf16 MFMA blocks: 4 column waves of two column tiles in one row group
    or two (64- and 128-row tiles, where LDS allows), and 4 waves of one
    column tile; ragged shapes (rows past M, columns past N, a last K step of
    32), one, two and four passes per step, zero-term sets cut short by the
    end of K or of a K split."""
    with lb.tuning(qmm_rgroups=int(rgroups), qmm_nt=int(nt)):
        for (M, N, K, group, bias) in [(128, 300, 416, 32, True), (100, 520, 1024, 64, False),
                                       (77, 257, 2080, 32, True), (128, 130, 2176, 128, False),
                                       (64, 200, 1280, 256, True), (120, 640, 4096, 128, True)]:
            run_small_linear(M, N, K, bits, group, "bf16", bias, lb.PATH_QMM, seed=bits + N)


# (M, N, K, group, bias, blocks): the qmm_blocks override sets the block target
# from which the schedule derives the K split (2 to 8 splits here; 0 = the
# default target).
SPLIT_SUM_CASES = [(128, 520, 2048, 64, True, 16), (100, 300, 4096, 128, False, 24),
                   (77, 257, 2080, 32, True, 9), (20, 300, 1024, 32, True, 24),
                   (128, 4096, 4096, 128, True, 0)]


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 5])
def test_qmm_forced_k_splits(bits, act):
    """K splits of 2 to 8 planes, from a workspace filled with garbage: within
    tolerance of the oracle and bitwise equal on a repeated call."""
    with lb.tuning(qmm_nt=2):    # the split counts above assume 2 column tiles
        _forced_k_splits(bits, act)


def _forced_k_splits(bits, act):
    for (M, N, K, group, bias, blocks) in SPLIT_SUM_CASES:
        case = Case("ss", M, K, N, bits, group, act, bias=bias, seed=bits + N + K)
        W = weight_for(case).numpy()
        ref = oracle.quantize(W, bits, group, act)
        x = make_x(case)
        b = make_bias(case)
        y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], group, bias_values(b))
        packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
        xd, bd = x.to(DEV), None if b is None else b.to(DEV)
        with lb.tuning(qmm_blocks=blocks):
            need = lb.lowbit_linear_workspace_bytes(bits, group, M, N, K, TORCH_ACT[act])
            assert need > 0, "the case must take a K split"
            ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
            y1 = lb.lowbit_linear(xd, packed, s, z, bd, bits, group, workspace=ws, path=lb.PATH_QMM)
            y2 = lb.lowbit_linear(xd, packed, s, z, bd, bits, group, workspace=ws, path=lb.PATH_QMM)
        torch.cuda.synchronize()
        what = f"M={M} N={N} K={K} b={bits} g={group} {act}"
        check_close(y1, y_ref, A, "K split " + what)
        assert torch.equal(y1, y2), "repeated call differs: " + what


def test_qmm_split_graph_replays():
    """A captured MFMA call with a K split (partial planes + reduce kernel):
    every replay, with eager work and synchronisation in between, matches the
    eager result bit for bit."""
    M, N, K, group, bits, act = 128, 4096, 4096, 128, 4, "bf16"
    case = Case("gr", M, K, N, bits, group, act, bias=True, seed=7)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, bits, group, act)
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
    xd, bd = make_x(case).to(DEV), make_bias(case).to(DEV)
    need = lb.lowbit_linear_workspace_bytes(bits, group, M, N, K, TORCH_ACT[act])
    assert need > 0
    ws = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    y_eager = lb.lowbit_linear(xd, packed, s, z, bd, bits, group, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            lb.lowbit_linear(xd, packed, s, z, bd, bits, group, y=y, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"graph replay {i} differs from the eager call"
        lb.lowbit_linear(xd, packed, s, z, bd, bits, group, workspace=ws)   # eager work between
        torch.cuda.synchronize()


def test_cached_workspace_survives_a_larger_call_between_graph_replays():
    """A graph captured over a call that took the binding's cached workspace
    keeps that buffer's address; a later, larger call on the same stream
    needs a bigger workspace.  The old buffer must stay alive: every replay
    after the larger call still matches the eager result bit for bit."""
    bits, group, act = 4, 128, "bf16"
    small = Case("ws_small", 128, 2048, 1024, bits, group, act, bias=True, seed=21)
    large = Case("ws_large", 128, 8192, 8192, bits, group, act, bias=False, seed=22)
    side = torch.cuda.Stream()

    def prepared(case):
        W = weight_for(case).numpy()
        ref = oracle.quantize(W, bits, group, act)
        packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
        b = make_bias(case)
        return make_x(case).to(DEV), packed, s, z, None if b is None else b.to(DEV)

    xs, ps, ss, zs, bs = prepared(small)
    xl, pl, sl, zl, bl = prepared(large)
    need_s = lb.lowbit_linear_workspace_bytes(bits, group, small.M, small.N, small.K, torch.bfloat16)
    need_l = lb.lowbit_linear_workspace_bytes(bits, group, large.M, large.N, large.K, torch.bfloat16)
    assert 0 < need_s < need_l, (need_s, need_l)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y_eager = lb.lowbit_linear(xs, ps, ss, zs, bs, bits, group)       # takes the cached workspace
        side.synchronize()
        y = torch.empty_like(y_eager)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            lb.lowbit_linear(xs, ps, ss, zs, bs, bits, group, y=y)
        side.synchronize()
        lb.lowbit_linear(xl, pl, sl, zl, bl, bits, group)                # needs a larger workspace
        side.synchronize()
        # memory handed out after the resize (the allocator would reuse a freed
        # workspace block for these sizes) must not be written by the replays
        sizes = [need_s, 1 << (need_s - 1).bit_length(), 1 << 20]
        sentinels = [torch.full((n,), 0x3C, dtype=torch.uint8, device=DEV) for n in sizes]
        for i in range(3):
            y.fill_(float("nan"))
            g.replay()
            side.synchronize()
            assert torch.equal(y, y_eager), f"replay {i} after a larger call differs"
            for t in sentinels:
                assert bool((t == 0x3C).all()), f"replay {i} wrote into memory it does not own"


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_qmm_small_m(bits, act):
    """The MFMA kernel with one or two 16-row tiles (M <= 32) on ragged
    shapes: rows past M, columns past N, a last K step of 32."""
    for (M, N, K, group, bias) in [(20, 300, 416, 32, True), (32, 257, 2080, 32, False),
                                   (3, 130, 160, 32, True), (9, 64, 4096, 128, False)]:
        run_small_linear(M, N, K, bits, group, act, bias, lb.PATH_QMM, seed=bits + M)


@pytest.mark.parametrize("bits", [2, 4, 6])
def test_qmm_without_workspace(bits):
    """With too little workspace the MFMA path runs without a K split (one
    block per tile over all of K)."""
    case = Case("nows", 96, 1536, 384, bits, 64, "f16", bias=True, seed=bits)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, bits, 64, "f16")
    x = make_x(case)
    b = make_bias(case)
    y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], 64, bias_values(b))
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, "f16")
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV)       # too small for any split
    y = lb.lowbit_linear(x.to(DEV), packed, s, z, b.to(DEV), bits, 64, workspace=tiny,
                         path=lb.PATH_QMM)
    torch.cuda.synchronize()
    check_close(y, y_ref, A, f"qmm without workspace b={bits}")


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [1, 4, 7])
def test_cross_path_m16(bits, act):
    case = Case("x", 16, 1024, 192, bits, 64, act, bias=True, seed=bits)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, bits, 64, act)
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
    x = make_x(case).to(DEV)
    b = make_bias(case).to(DEV)
    y1 = lb.lowbit_linear(x, packed, s, z, b, bits, 64, path=lb.PATH_QMV)
    y2 = lb.lowbit_linear(x, packed, s, z, b, bits, 64, path=lb.PATH_QMM)
    y3 = lb.lowbit_linear(x, packed, s, z, b, bits, 64)
    torch.cuda.synchronize()
    y_ref, A = oracle.linear(x_values(x.cpu()), ref["q"], ref["s"], ref["z"], 64,
                             bias_values(b.cpu()))
    check_close(y1, y_ref, A, "qmv")
    check_close(y2, y_ref, A, "qmm")
    assert torch.equal(y3, y2)    # M = 16 takes the MFMA path by default


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", range(1, 8))
def test_exact_integer_bitexact(bits, act):
    """s = 1, z = -2^(b-1), x in {-1,0,1}: all partial sums are exact integers,
    so y must equal the oracle's value rounded once to the activation dtype."""
    rng = np.random.default_rng(bits * 3 + len(act))
    group = 64
    paths = [lb.PATH_QMV] + ([lb.PATH_QMM] if act != "f32" else [])
    for M, N, K in [(1, 96, 4096), (4, 40, 1024), (16, 72, 2048), (33, 50, 512)]:
        q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
        s = np.ones((N, K // group), np.float32)
        z = np.full((N, K // group), -(1 << (bits - 1)), np.float32)
        xv = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
        bv = rng.integers(-8, 9, size=N).astype(np.float32)
        y_ref, _ = oracle.linear(xv, q, s, z, group, bv)
        assert np.abs(y_ref).max() < 65504
        expect = oracle.round_to_storage(y_ref.astype(np.float32), act)[1]
        packed, s_t, z_t = upload_quant(q, s, z, bits, act)
        x = torch.from_numpy(xv).to(TORCH_ACT[act]).to(DEV)
        b = torch.from_numpy(bv).to(TORCH_ACT[act]).to(DEV)
        for path in paths:
            y = lb.lowbit_linear(x, packed, s_t, z_t, b, bits, group, path=path)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(act_bits(y), expect, err_msg=f"M={M} path={path}")


@pytest.mark.parametrize("path", [lb.PATH_QMV, lb.PATH_QMM])
def test_one_hot_positions(path):
    """x = e_k picks one dequantized weight: pins the unpack position mapping."""
    bits, group, N, K, act = 7, 32, 24, 256, "f16"
    case = Case("o", 1, K, N, bits, group, act, seed=5)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, bits, group, act)
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], bits, act)
    x = torch.eye(K, dtype=torch.float16)
    y = lb.lowbit_linear(x.to(DEV), packed, s, z, None, bits, group, path=path)
    torch.cuda.synchronize()
    y_ref, A = oracle.linear(x.float().numpy(), ref["q"], ref["s"], ref["z"], group)
    check_close(y, y_ref, A, f"one-hot path={path}")


def test_determinism_and_m0():
    case = Case("d", 3, 4096, 512, 3, 64, "f16", bias=True, seed=2)
    W = weight_for(case).numpy()
    ref = oracle.quantize(W, 3, 64, "f16")
    packed, s, z = upload_quant(ref["q"], ref["s"], ref["z"], 3, "f16")
    x = make_x(case).to(DEV)
    b = make_bias(case).to(DEV)
    for path in (lb.PATH_QMV, lb.PATH_QMM):
        ys = [lb.lowbit_linear(x, packed, s, z, b, 3, 64, path=path) for _ in range(5)]
        torch.cuda.synchronize()
        for y in ys[1:]:
            assert torch.equal(act_bits_t(y), act_bits_t(ys[0]))
    y0 = lb.lowbit_linear(x[:0], packed, s, z, b, 3, 64)
    assert y0.shape == (0, 512)


def act_bits_t(t):
    return t.view(torch.int16)


# --------------------------------------------- workloads at full size --

def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    rows = set([0, 1, N - 2, N - 1]) | set(rng.choice(N, size=min(N, 44), replace=False).tolist())
    return np.array(sorted(rows))


CASES = all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_workload_sampled(case):
    """Full-size workload, default dispatch: GPU quantize -> GPU linear; the
    oracle recomputes sampled rows from scratch."""
    W = weight_for(case)
    x = make_x(case)
    b = make_bias(case)
    packed, s, z, _ = gpu_quantize(W, case.bits, case.group, case.act, want_codes=False)
    y = lb.lowbit_linear(x.to(DEV), packed, s, z, None if b is None else b.to(DEV), case.bits,
                         case.group)
    torch.cuda.synchronize()
    rows = _sample_rows(case.N, zlib.crc32(case.name.encode()) % 1000)
    ref = oracle.quantize(W.numpy()[rows], case.bits, case.group, case.act)
    assert_quant_equal(ref, packed, s, z, None, case.bits, rows=rows)
    y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], case.group,
                             None if b is None else bias_values(b)[rows])
    check_close(y[:, torch.from_numpy(rows).to(DEV)], y_ref, A, case.name)


def random_shape_cases(chunk: int, count: int = 12):
    """Seeded random shapes: M from 1 to 160 (both kernels and the crossover),
    N from 1 to 1500 (ragged row groups and column tiles), K up to 4096 in
    whole groups (one to many K steps, K splits, one and two rounds per
    lane), every width, group, activation type and bias choice."""
    rng = np.random.default_rng(0x5EED + chunk)
    cases = []
    for i in range(count):
        act = ["f32", "f16", "bf16"][int(rng.integers(3))]
        m_band = int(rng.integers(3))
        M = int(rng.integers(1, 7)) if m_band == 0 else (int(rng.integers(7, 41)) if m_band == 1
                                                         else int(rng.integers(41, 161)))
        if act == "f32":
            M = min(M, 8)
        group = [32, 64, 128, 256][int(rng.integers(4))]
        K = group * int(rng.integers(1, 4096 // group + 1))
        N = int(rng.integers(1, 1501))
        bits = int(rng.integers(1, 8))
        cases.append(Case(f"rnd{chunk}_{i}", M, K, N, bits, group, act,
                          bias=bool(rng.integers(2)), seed=1000 * chunk + i))
    return cases


@pytest.mark.parametrize("chunk", range(12))
def test_random_shapes(chunk):
    """GPU quantizer bit-exact and the linear within tolerance of the oracle,
    on the default path and on every forced path the activation type allows,
    for seeded random shapes."""
    for case in random_shape_cases(chunk):
        what = (f"{case.name}: M={case.M} N={case.N} K={case.K} b={case.bits} "
                f"g={case.group} {case.act} bias={case.bias}")
        W = weight_for(case)
        ref = oracle.quantize(W.numpy(), case.bits, case.group, case.act)
        packed, s, z, codes = gpu_quantize(W, case.bits, case.group, case.act)
        torch.cuda.synchronize()
        assert_quant_equal(ref, packed, s, z, codes, case.bits)
        x = make_x(case)
        b = make_bias(case)
        y_ref, A = oracle.linear(x_values(x), ref["q"], ref["s"], ref["z"], case.group,
                                 bias_values(b))
        xd = x.to(DEV)
        bd = None if b is None else b.to(DEV)
        paths = [lb.PATH_AUTO, lb.PATH_QMV] + ([lb.PATH_QMM] if case.act != "f32" else [])
        for path in paths:
            y = lb.lowbit_linear(xd, packed, s, z, bd, case.bits, case.group, path=path)
            torch.cuda.synchronize()
            check_close(y, y_ref, A, f"{what} path={path}")
