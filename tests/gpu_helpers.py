"""Shared helpers for the GPU parity tests (inputs from the seeded generators,
expected values from the CPU oracle, results from the HIP library)."""
import functools

import numpy as np
import torch

import oracle
from bit_groupwise_weight_amd import lowbit
from bit_groupwise_weight_amd.workloads import Case, make_bias, make_weight, make_x

DEV = torch.device("cuda:0")
TORCH_ACT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def act_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU/GPU tensor of an activation dtype."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def cached_weight(N, K, seed, w_std, w_row_loguniform):
    c = Case("w", 1, K, N, 4, 32, "f32", w_std=w_std, w_row_loguniform=w_row_loguniform, seed=seed)
    return make_weight(c)


def weight_for(case: Case) -> torch.Tensor:
    return cached_weight(case.N, case.K, case.seed, case.w_std, case.w_row_loguniform)


def upload_quant(q, s, z, bits, act):
    """Oracle-quantized weights -> device tensors in the library's format."""
    packed = torch.from_numpy(oracle.pack(q, bits)).to(DEV)
    s_t = torch.from_numpy(np.ascontiguousarray(s)).to(TORCH_ACT[act]).to(DEV)
    z_t = torch.from_numpy(np.ascontiguousarray(z)).to(TORCH_ACT[act]).to(DEV)
    return packed, s_t, z_t


# (label, worst err/tol) of every comparison in this session, printed by the
# terminal summary of tests/conftest.py
ERR_TOL_LOG = []


def check_close(y_gpu: torch.Tensor, y_ref: np.ndarray, A: np.ndarray, what: str):
    y = y_gpu.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(y - y_ref)
    tol = oracle.tolerance(A)
    bad = err > tol
    ratio = float((err / tol).max()) if err.size else 0.0
    ERR_TOL_LOG.append((what, ratio))
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; worst "
                           f"err {err.max():.3e} (tol there {tol.flat[int(err.argmax())]:.3e})")
    return ratio


def x_values(x: torch.Tensor) -> np.ndarray:
    return x.float().numpy()


def bias_values(b):
    return None if b is None else b.float().numpy()
