"""GPU precision stress: inputs chosen to expose rounding that random,
zero-mean data hides, each compared with the fp64 oracle against
1e-3 + 2e-3 * sum_k |x_k w_k| (w the dequantized weight).

Families:
  * large activations (standard deviation 300, fp16 and bf16) on ordinary
    weights -- the absolute floor of the tolerance no longer hides errors;
  * groups of exact zeros with one outlier weight (positive: z = 0 and every
    other code 0; negative: z = the outlier and every other code 2^b - 1, so
    s*q and z nearly cancel), with large activations;
  * the same with an exact grid (s * (2^b - 1) == -z exactly), where the zeros
    reconstruct to exactly 0;
  * correlated rounding of the dequantized weight: every weight of a row
    rounds the same way if it is first rounded to the activation type
    (z = +1 / -1.0078125 alternating, s = 2^-8 - 2^-16, q = 1, x = 1).

Every decode and MFMA path the activation type allows runs on each input.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_groupwise_weight_amd import lowbit as lb
from tests.gpu_helpers import DEV, TORCH_ACT, check_close, upload_quant

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module", autouse=True)
def _lib(lowbit_lib):
    return lowbit_lib


def paths_for(act, M):
    out = [("qmv", lb.PATH_QMV)]
    if act != "f32":
        out.append(("qmm", lb.PATH_QMM))
    return out


def run_paths(x32, q, s, z, bias32, bits, group, act, label, skip=()):
    """Oracle vs every path (but those named in skip); x32/bias32 are fp32
    arrays already exact in act."""
    y_ref, A = oracle.linear(x32, q, s, z, group, bias32)
    packed, s_t, z_t = upload_quant(q, s, z, bits, act)
    xd = torch.from_numpy(x32).to(TORCH_ACT[act]).to(DEV)
    bd = None if bias32 is None else torch.from_numpy(bias32).to(TORCH_ACT[act]).to(DEV)
    worst = 0.0
    for name, path in paths_for(act, x32.shape[0]):
        if name in skip:
            continue
        y = lb.lowbit_linear(xd, packed, s_t, z_t, bd, bits, group, path=path)
        torch.cuda.synchronize()
        worst = max(worst, check_close(y, y_ref, A, f"{label} {name}"))
    return worst


def act_round(a, act):
    return oracle.round_to_storage(np.asarray(a, np.float32), act)[0]


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bits,group", [(1, 32), (4, 128), (7, 64), (3, 256)])
@pytest.mark.parametrize("M", [1, 3, 20])
def test_large_activations(bits, group, M, act):
    if act == "f32" and M > 4:
        pytest.skip("fp32 activations run the decode kernel at small M only")
    rng = np.random.default_rng(bits * 100 + group + M)
    N, K = 136, 2048
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ref = oracle.quantize(W, bits, group, act)
    x = act_round(rng.standard_normal((M, K)) * 300.0, act)
    run_paths(x, ref["q"], ref["s"], ref["z"], None, bits, group, act,
              f"large-x M={M} b={bits} g={group} {act}")


def zero_dominated(N, K, group, seed, sign):
    """Weights that are exact zeros except one outlier per group."""
    rng = np.random.default_rng(seed)
    W = np.zeros((N, K), np.float32)
    G = K // group
    pos = rng.integers(0, group, size=(N, G))
    mag = (np.abs(rng.standard_normal((N, G))) * 0.05 + 0.01).astype(np.float32)
    cols = (np.arange(G)[None, :] * group + pos)
    W[np.arange(N)[:, None], cols] = sign * mag
    return W


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("bits", [1, 4, 7])
@pytest.mark.parametrize("M", [1, 4, 24])
def test_zero_groups_with_outlier(bits, sign, M, act):
    if act == "f32" and M > 4:
        pytest.skip("fp32 activations run the decode kernel at small M only")
    group, N, K = 64, 72, 4096
    W = zero_dominated(N, K, group, seed=bits * 7 + M, sign=sign)
    ref = oracle.quantize(W, bits, group, act)
    rng = np.random.default_rng(bits + M)
    x = act_round(rng.standard_normal((M, K)) * 300.0, act)
    run_paths(x, ref["q"], ref["s"], ref["z"], None, bits, group, act,
              f"zero-groups sign={sign:+.0f} M={M} b={bits} {act}")


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 7])
def test_exact_grid_cancellation(bits, act):
    """s * qmax == -z exactly (powers of two), so code qmax reconstructs to
    exactly 0: the zeros of each group take code qmax and the group's one
    nonzero weight (-qmax * s) code 0.  Activations are large everywhere,
    including at the nonzero weights."""
    rng = np.random.default_rng(bits)
    qmax = (1 << bits) - 1
    group, N, K, M = 32, 40, 1024, 4
    G = K // group
    e = rng.integers(-9, -4, size=(N, G)).astype(np.float64)
    s = (2.0 ** e).astype(np.float32)
    z = (-qmax * 2.0 ** e).astype(np.float32)
    q = np.full((N, K), qmax, np.uint8)
    pos = rng.integers(0, group, size=(N, G))
    q[np.arange(N)[:, None], np.arange(G)[None, :] * group + pos] = 0
    x = act_round(rng.standard_normal((M, K)) * 300.0, act)
    run_paths(x, q, s, z, None, bits, 32, act, f"exact-grid cancel b={bits} {act}")


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_correlated_weight_rounding(M, act):
    """Dequantized weights 1 + s and -1.0078125 + s (s = 2^-8 - 2^-16): in
    bf16 every one of them rounds the same way, so a kernel that rounds s*q + z
    to bf16 before multiplying is off by ~2^-8 * sum |x*w| (twice the
    tolerance).  Exact codes with s and z applied in fp32 are exact here."""
    bits, group, N, K = 4, 32, 48, 4096
    G = K // group
    s = np.full((N, G), 2.0 ** -8 - 2.0 ** -16, np.float32)
    z = np.where(np.arange(G) % 2 == 0, 1.0, -1.0078125).astype(np.float32)[None, :].repeat(N, 0)
    q = np.ones((N, K), np.uint8)
    x = np.ones((M, K), np.float32)
    run_paths(x, q, s, z, None, bits, group, act, f"correlated-rounding M={M} {act}")


@pytest.mark.parametrize("bits,group", [(1, 64), (4, 32), (7, 128)])
@pytest.mark.parametrize("M", [1, 3, 24])
def test_fp16_near_max_activations(bits, group, M):
    """fp16 activations near +-6e4 (close to the fp16 maximum) in a few
    groups, ordinary ones elsewhere, on small weights so that y stays in
    range: the products x*q and the group sums are far larger than anywhere
    else, and every path must keep them exact enough."""
    rng = np.random.default_rng(bits * 31 + M + group)
    N, K = 96, 2048
    W = (rng.standard_normal((N, K)) * 1e-4).astype(np.float32)
    ref = oracle.quantize(W, bits, group, "f16")
    x = rng.standard_normal((M, K))
    for gi in rng.choice(K // group, size=3, replace=False):
        sign = np.where(rng.random((M, group)) < 0.5, -1.0, 1.0)
        x[:, gi * group:(gi + 1) * group] = sign * rng.uniform(3e4, 6e4, size=(M, group))
    x = act_round(x, "f16")
    run_paths(x, ref["q"], ref["s"], ref["z"], None, bits, group, "f16",
              f"near-max x M={M} b={bits} g={group} f16")
