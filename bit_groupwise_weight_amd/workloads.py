"""Seeded synthetic inputs for the groupwise low-bit linear layer.

This module only draws random tensors and casts them to the activation dtype.
It contains none of the method's arithmetic (no quantization, packing or
dequantization), so both the CPU oracle (test infrastructure) and the HIP path
can be fed from it without sharing any of the computation.

The shapes, distributions and parameter ranges follow the workloads the pages
describe:
  * bit widths 1..7 and group sizes 32/64/128/256 -- "Add torchao mps ops",
    the description of the linear:afpwx scheme;
  * Llama 3.1-8B / 3.2-1B / 3.2-3B decode at batch 1, group 64, fp16
    activations -- "metal lowbit kernels: qmv_fast optimization",
    Performance Improvement tables;
  * int4 weight-only, group 128, bf16, batch 1 and 128 -- "Add support for
    fbgemm int4 mm kernel", H100 table;
  * fp32 activations -- "[MPS] Add support for Int4 groupwise quantization",
    the export command (-d fp32, -G 32).
The trained checkpoints those pages run are not available; synthetic tensors of
the same linear-layer shapes stand in for them.

Seeds: every case uses base seed 0 with separate generators per tensor:
W = seed, x = seed + 1, bias = seed + 2, outlier mask = seed + 3,
per-row weight scale = seed + 4.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import numpy as np
import torch

ACT_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Case:
    """One linear-layer workload: y[M,N] = x[M,K] . dequant(Wq)[N,K]^T (+ bias)."""

    name: str
    M: int
    K: int
    N: int
    bits: int
    group: int
    act: str                    # "f32" | "f16" | "bf16"; also the scale/zero dtype
    bias: bool = False
    w_std: float = 0.02         # W ~ N(0, w_std) unless w_row_loguniform is set
    w_row_loguniform: Optional[tuple] = None   # (lo, hi): sigma_n log-uniform per row
    x_outlier_frac: float = 0.0  # iid Bernoulli mask over x entries ...
    x_outlier_mult: float = 1.0  # ... whose entries are multiplied by this
    bias_std: float = 0.1
    seed: int = 0

    @property
    def num_groups(self) -> int:
        return self.K // self.group


def _normal_f32(seed: int, shape) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_act(a32: np.ndarray, act: str) -> torch.Tensor:
    """Round an fp32 array to the activation dtype (torch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(ACT_DTYPES[act])


def make_weight(case: Case) -> torch.Tensor:
    """W[N, K] fp32."""
    w = _normal_f32(case.seed, (case.N, case.K))
    if case.w_row_loguniform is not None:
        lo, hi = case.w_row_loguniform
        rng = np.random.default_rng(case.seed + 4)
        sigma = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(case.N, 1))).astype(np.float32)
        w *= sigma
    else:
        w *= np.float32(case.w_std)
    return torch.from_numpy(w)


def make_x(case: Case) -> torch.Tensor:
    """x[M, K] in the activation dtype, drawn in fp32 and rounded to nearest even."""
    x = _normal_f32(case.seed + 1, (case.M, case.K))
    if case.x_outlier_frac > 0.0:
        rng = np.random.default_rng(case.seed + 3)
        mask = rng.random(size=x.shape) < case.x_outlier_frac
        x = np.where(mask, x * np.float32(case.x_outlier_mult), x).astype(np.float32)
    return to_act(x, case.act)


def make_bias(case: Case) -> Optional[torch.Tensor]:
    if not case.bias:
        return None
    b = _normal_f32(case.seed + 2, (case.N,)) * np.float32(case.bias_std)
    return to_act(b, case.act)


def make_inputs(case: Case) -> Dict[str, Optional[torch.Tensor]]:
    """CPU tensors for one case: W fp32 [N,K], x act [M,K], bias act [N] or None."""
    return {"W": make_weight(case), "x": make_x(case), "bias": make_bias(case)}


def input_hash(inputs: Dict[str, Optional[torch.Tensor]]) -> str:
    h = hashlib.sha256()
    for k in sorted(inputs):
        t = inputs[k]
        if t is None:
            continue
        h.update(k.encode())
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- workloads --

def single_qmv() -> List[Case]:
    """Single decode linear: M=1, K=N=2048, 4-bit, group 64, fp32 activations."""
    return [Case("single_k2048_n2048_b4_g64_f32", 1, 2048, 2048, 4, 64, "f32")]


LLAMA31_8B_SHAPES = [(4096, 4096), (4096, 14336), (14336, 4096), (4096, 1024)]


def llama8b_decode() -> List[Case]:
    """Llama-3.1-8B-shaped decode linears, M=1, fp16, group 64, bits 1..7."""
    out = []
    for (K, N) in LLAMA31_8B_SHAPES:
        for b in range(1, 8):
            out.append(Case(f"llama8b_k{K}_n{N}_b{b}_g64", 1, K, N, b, 64, "f16"))
    return out


LLAMA32_SMALL_SHAPES = [(2048, 8192), (8192, 2048), (3072, 8192), (8192, 3072)]


def llama_small_decode() -> List[Case]:
    """Llama-3.2-1B/3B-shaped decode linears, M=1, fp16 with bias, groups 32/256."""
    out = []
    for (K, N) in LLAMA32_SMALL_SHAPES:
        for g in (32, 256):
            for b in (3, 5, 6, 7):
                out.append(Case(f"llama_small_k{K}_n{N}_b{b}_g{g}", 1, K, N, b, g, "f16", bias=True))
    return out


def batched_qmm() -> List[Case]:
    """Batched MFMA path: M=128, 4-bit, group 128, bf16 activations."""
    return [Case(f"batched_m128_k{K}_n{N}_b4_g128", 128, K, N, 4, 128, "bf16")
            for (K, N) in [(4096, 14336), (14336, 4096)]]


def mixed_sweep() -> List[Case]:
    """M in {1,4,16,64}, K=N=4096, bits {1,2,4,7}, groups {32..256}; fp16 x with
    1% outliers x20, per-row weight scale log-uniform in [0.005, 0.05], bias on."""
    out = []
    for M in (1, 4, 16, 64):
        for b in (1, 2, 4, 7):
            for g in (32, 64, 128, 256):
                out.append(Case(f"mixed_m{M}_b{b}_g{g}", M, 4096, 4096, b, g, "f16", bias=True,
                                w_row_loguniform=(0.005, 0.05), x_outlier_frac=0.01,
                                x_outlier_mult=20.0))
    return out


def activation_quantized() -> List[Case]:
    """The activation-quantized variant (8-bit dynamic activations with 4-bit
    weights in groups of 32, the export mode of "[MPS] Add support for Int4
    groupwise quantization") at the batched Llama-3.1-8B MLP shapes: M=128,
    bf16 activations x ~ N(0,1), W ~ N(0,0.02).  Not part of WORKLOADS: these
    cases run through the int8-activation entry points, not lowbit_linear."""
    return [Case(f"a8_m128_k{K}_n{N}_b4_g32", 128, K, N, 4, 32, "bf16")
            for (K, N) in [(4096, 14336), (14336, 4096)]]


WORKLOADS = {
    "single_qmv": single_qmv,
    "llama8b_decode": llama8b_decode,
    "llama_small_decode": llama_small_decode,
    "batched_qmm": batched_qmm,
    "mixed_sweep": mixed_sweep,
}


def all_cases() -> List[Case]:
    out: List[Case] = []
    for f in WORKLOADS.values():
        out.extend(f())
    return out
