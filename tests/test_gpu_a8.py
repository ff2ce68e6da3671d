"""GPU parity of the activation-quantized variant (8-bit dynamic activations
with groupwise low-bit weights) against the CPU oracle, through the C ABI.

The activation quantizer must match the oracle bit for bit (codes and the
fp32 scale of every row); the linear must be within the layer's tolerance,
1e-3 + 2e-3 * sum_k |a_m xq[m, k] w[n, k]|, of the oracle's fp64 result.
Inputs come from the seeded generators; weights are quantized and packed by
the oracle, and the linear's int8 inputs by the oracle too (the end-to-end
cases chain the two GPU calls).
"""
import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit
from bit_groupwise_weight_amd.workloads import Case, activation_quantized, make_weight, make_x, to_act
from tests.gpu_helpers import DEV, TORCH_ACT, check_close, upload_quant

pytestmark = pytest.mark.gpu


def x_rows(M, K, act, seed, special=True):
    """fp32 values of seeded activations in `act` (1 % outliers x20); with
    `special`, row 1 is zero, row 2 holds exact ties of a unit scale (max 127,
    values k + 1/2) and row 3 a tiny scale."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random((M, K)) < 0.01] *= 20.0
    if special and M >= 4:
        x[1] = 0.0
        k = rng.integers(-127, 127, size=K)
        x[2] = k + 0.5
        x[2, 0] = 127.0
        x[3] *= np.float32(1e-3)
    return to_act(x, act)


def quant_weights(N, K, bits, group, act, seed):
    W = make_weight(Case("w", 1, K, N, bits, group, act, seed=seed)).numpy()
    r = oracle.quantize(W, bits, group, act)
    packed, s, z = upload_quant(r["q"], r["s"], r["z"], bits, act)
    return r, packed, s, z


def bias_for(N, act, seed):
    rng = np.random.default_rng(seed + 2)
    return to_act((rng.standard_normal(N) * 0.1).astype(np.float32), act)


def check_quantizer(x_dev, x_cpu):
    xq, a = lowbit.lowbit_quantize_act_i8(x_dev)
    xq_ref, a_ref = oracle.quantize_activations_i8(x_cpu.float().numpy())
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    a_gpu = a.cpu().numpy()
    assert np.array_equal(np.isnan(a_gpu), np.isnan(a_ref))
    fin = ~np.isnan(a_ref)
    np.testing.assert_array_equal(a_gpu[fin].view(np.uint32), a_ref[fin].view(np.uint32))
    return xq, a, xq_ref, a_ref


# ------------------------------------------------------------- quantizer --

@pytest.mark.parametrize("act", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (7, 4096), (128, 4096), (3, 14336), (2, 8224)])
def test_act_quant_bit_exact(act, M, K):
    x = x_rows(M, K, act, seed=M + K)
    check_quantizer(x.to(DEV), x)


def test_act_quant_ties_at_a_scale_that_is_not_a_power_of_two():
    # fp32 rows: max 127 c 2^-10 gives a = c 2^-10; (2k + 1) c 2^-11 are ties
    rows = []
    for c in (3, 255, 61):
        ks = np.arange(-127, 127)
        r = np.concatenate([[127.0 * c * 2.0 ** -10], (2 * ks + 1) * c * 2.0 ** -11])
        rows.append(np.resize(r, 288))
    x = torch.from_numpy(np.array(rows, np.float32))
    xq, _, _, _ = check_quantizer(x.to(DEV), x)
    assert xq.abs().max().item() == 127


@pytest.mark.parametrize("act", ["bf16", "f16", "f32"])
def test_act_quant_nonfinite_and_zero_rows(act):
    x = x_rows(6, 256, act, seed=5, special=False)
    x[0] = 0
    x[1, 17] = float("nan")
    x[2, 255] = float("inf")
    x[3, 0] = float("-inf")
    x[4, 100] = -0.0
    xq, a, _, _ = check_quantizer(x.to(DEV), x)
    a = a.cpu()
    assert a[0].item() == 0 and not xq[0].any()
    for m in (1, 2, 3):
        assert torch.isnan(a[m]) and not xq[m].any()
    assert not torch.isnan(a[4]) and not torch.isnan(a[5])


# ---------------------------------------------------------------- linear --

def run_linear_case(M, N, K, bits, group, act, seed, bias=True, mtt=None, nt=None):
    r, packed, s, z = quant_weights(N, K, bits, group, act, seed)
    x = x_rows(M, K, act, seed + 1)
    xq_ref, a_ref = oracle.quantize_activations_i8(x.float().numpy())
    if M >= 5:
        a_ref = a_ref.copy()
        a_ref[4] = np.float32(np.nan)          # a row that held a NaN
        xq_ref[4] = 0
    b = bias_for(N, act, seed) if bias else None
    y_ref, A = oracle.linear_a8(xq_ref, a_ref, r["q"], r["s"], r["z"], group,
                                None if b is None else b.float().numpy())
    xq_d = torch.from_numpy(xq_ref).to(DEV)
    a_d = torch.from_numpy(a_ref).to(DEV)
    b_d = None if b is None else b.to(DEV)
    with lowbit.tuning(a8_mtt=mtt or 0, a8_nt=nt or 0):
        y = lowbit.lowbit_linear_a8(xq_d, a_d, packed, s, z, b_d, bits, group)
    torch.cuda.synchronize()
    nan_rows = np.isnan(a_ref)
    yc = y.float().cpu()
    assert torch.isnan(yc[torch.from_numpy(nan_rows)]).all()
    keep = ~nan_rows
    label = f"a8 b{bits} g{group} {act} M={M} N={N} K={K} mtt={mtt} nt={nt}"
    check_close(y[torch.from_numpy(keep).to(DEV)], y_ref[keep], A[keep], label)
    return y


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_linear_a8_every_width_and_group(bits, group):
    # ragged M and N; K with a half window at group 32 (K = 64 w + 32)
    K = {32: 416, 64: 448, 128: 384, 256: 512}[group]
    act = ["bf16", "f16", "f32"][(bits + group // 32) % 3]
    for mtt in (1, 2, 4):
        for nt in (1, 2):
            run_linear_case(37, 200, K, bits, group, act, seed=bits * 10 + group, mtt=mtt, nt=nt)


@pytest.mark.parametrize("act", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits,group", [(4, 32), (3, 64), (7, 32)])
def test_linear_a8_dtypes(act, bits, group):
    run_linear_case(20, 96, 2048 + 32 * (group == 32), bits, group, act, seed=3, bias=act != "f32")


@pytest.mark.parametrize("group", [64, 128, 256])
@pytest.mark.parametrize("act", ["bf16", "f16", "f32"])
def test_linear_a8_batched_scales(group, act):
    # an even number of groups and many batches: the scales and zeros of a
    # batch come in one load, from an even start slot for 2-byte values
    for mtt in (1, 2, 4):
        for nt in (1, 2):
            run_linear_case(37, 150, 3072, 4, group, act, seed=group + mtt, mtt=mtt, nt=nt)


@pytest.mark.parametrize("M", [1, 2, 16, 17, 64, 129])
def test_linear_a8_row_counts(M):
    run_linear_case(M, 130, 1024, 4, 32, "bf16", seed=M)


def test_linear_a8_end_to_end_small():
    # GPU quantizer -> GPU linear, against oracle quantizer -> oracle linear
    M, N, K, bits, group, act = 24, 300, 1056, 4, 32, "bf16"
    r, packed, s, z = quant_weights(N, K, bits, group, act, 9)
    x = x_rows(M, K, act, 10)
    xq, a, xq_ref, a_ref = check_quantizer(x.to(DEV), x)
    b = bias_for(N, act, 9)
    y = lowbit.lowbit_linear_a8(xq, a, packed, s, z, b.to(DEV), bits, group)
    y_ref, A = oracle.linear_a8(xq_ref, a_ref, r["q"], r["s"], r["z"], group, b.float().numpy())
    keep = a_ref != 0
    assert torch.equal(y[1].cpu(), b)                        # the zero row: bias exactly
    check_close(y[torch.from_numpy(keep).to(DEV)], y_ref[keep], A[keep], "a8 end-to-end small")


@pytest.mark.parametrize("case", activation_quantized(), ids=lambda c: c.name)
def test_linear_a8_full_size(case):
    # every output of the batched Llama-3.1-8B MLP shapes, in the launch the
    # benchmark times; twice, bitwise equal
    x = make_x(case)
    r, packed, s, z = quant_weights(case.N, case.K, case.bits, case.group, case.act, case.seed)
    xq, a, xq_ref, a_ref = check_quantizer(x.to(DEV), x)
    y1 = lowbit.lowbit_linear_a8(xq, a, packed, s, z, None, case.bits, case.group)
    y2 = lowbit.lowbit_linear_a8(xq, a, packed, s, z, None, case.bits, case.group)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y_ref, A = oracle.linear_a8(xq_ref, a_ref, r["q"], r["s"], r["z"], case.group)
    check_close(y1, y_ref, A, f"a8 full {case.name}")


def test_linear_a8_graph_replay():
    # captured once, replayed three times with eager work in between
    M, N, K, bits, group, act = 64, 512, 1024, 4, 32, "bf16"
    _, packed, s, z = quant_weights(N, K, bits, group, act, 4)
    x = x_rows(M, K, act, 4, special=False).to(DEV)
    xq, a = lowbit.lowbit_quantize_act_i8(x)
    y_eager = lowbit.lowbit_linear_a8(xq, a, packed, s, z, None, bits, group)
    y = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        lowbit.lowbit_quantize_act_i8(x, xq, a, stream=stream)
        with torch.cuda.graph(g, stream=stream):
            lowbit.lowbit_quantize_act_i8(x, xq, a, stream=stream)
            lowbit.lowbit_linear_a8(xq, a, packed, s, z, None, bits, group, y=y, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
