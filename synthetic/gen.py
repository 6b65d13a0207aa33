"""Seeded Gaussian Q/K/V for the five benchmark workloads and for small test cases.

Recipe (the same for every workload; only the sizes and the K offset law differ):

* generator: ``numpy.random.default_rng(seed)`` (PCG64), draws in float32;
* draw order: Q noise, K noise, K per-channel offset, outlier channel indices,
  V noise;
* Q ~ N(0, 1) and V ~ N(0, 1), element-wise;
* K = N(0, 1) noise + an offset that is constant over tokens for each
  (batch, kv head, channel), drawn from N(0, sigma^2); for the Llama-shaped
  workloads, 4 seeded channels per (batch, kv head) have their offset scaled
  by 20 (large per-channel outliers that the K smoothing step has to absorb);
* the float32 values are cast once, round-to-nearest-even, to the input dtype
  (float16 or bfloat16) with torch's CPU cast.

The outputs are CPU torch tensors in the input dtype, laid out [B, H, N, d]
row-major. Nothing in this module performs any step of the attention method.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np
import torch

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Problem:
    """Shape, dtype, masking mode and input law of one attention problem."""

    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "f16" or "bf16"
    causal: bool
    sparse: Optional[Tuple[int, int]] = None  # (keep_num, keep_den) or dense
    k_offset_std: float = 2.0
    outliers: int = 0
    outlier_scale: float = 20.0
    name: str = ""

    @property
    def torch_dtype(self):
        return _TORCH_DTYPES[self.dtype]

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


# The five workloads. Block sizes of the sparse workload (query block 128,
# KV block 64) are the library's fixed quantization blocks.
CONFIGS = {
    1: Problem(1, 2, 2, 256, 64, "f16", False, None, 2.0, 0, 20.0,
               "tiny non-causal B1 H2 N256 d64 fp16"),
    2: Problem(1, 32, 8, 8192, 128, "bf16", True, None, 3.0, 4, 20.0,
               "Llama-3.1-8B-shaped causal prefill B1 Hq32 Hkv8 N8192 d128 bf16"),
    3: Problem(2, 24, 24, 4096, 64, "f16", False, None, 2.0, 0, 20.0,
               "non-causal vision/diffusion B2 H24 N4096 d64 fp16"),
    4: Problem(1, 32, 8, 65536, 128, "bf16", True, None, 3.0, 4, 20.0,
               "long-context causal prefill B1 Hq32 Hkv8 N65536 d128 bf16"),
    5: Problem(1, 32, 8, 32768, 128, "bf16", True, (1, 10), 3.0, 4, 20.0,
               "block-sparse causal prefill B1 Hq32 Hkv8 N32768 d128 bf16, keep first+diagonal+top 10%"),
}


def config_problem(c: int) -> Problem:
    return CONFIGS[c]


def _draw(p: Problem, seed: int):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((p.B, p.Hq, p.N, p.d), dtype=np.float32)
    k = rng.standard_normal((p.B, p.Hkv, p.N, p.d), dtype=np.float32)
    off = rng.standard_normal((p.B, p.Hkv, 1, p.d), dtype=np.float32)
    off *= np.float32(p.k_offset_std)
    for b in range(p.B):
        for h in range(p.Hkv):
            if p.outliers:
                idx = rng.choice(p.d, size=p.outliers, replace=False)
                off[b, h, 0, idx] *= np.float32(p.outlier_scale)
    k += off
    v = rng.standard_normal((p.B, p.Hkv, p.N, p.d), dtype=np.float32)
    return q, k, v


def make_problem_inputs(p: Problem, seed: int):
    """Draw Q, K, V for problem ``p`` and cast them to its dtype."""
    q, k, v = _draw(p, seed)
    dt = p.torch_dtype
    out = {
        "q": torch.from_numpy(q).to(dt),
        "k": torch.from_numpy(k).to(dt),
        "v": torch.from_numpy(v).to(dt),
    }
    del q, k, v
    return out


def make_config(c: int, seed: Optional[int] = None, N: Optional[int] = None):
    """Inputs of workload ``c`` (1..5); default seed is 1000 + c.

    ``N`` optionally shortens the sequence (same law, same seed) for tests that
    need the workload's distribution at a size the oracle finishes quickly.
    Returns (problem, {"q","k","v"}).
    """
    p = CONFIGS[c]
    if N is not None:
        p = replace(p, N=N)
    if seed is None:
        seed = 1000 + c
    return p, make_problem_inputs(p, seed)


def make_case(B=1, Hq=2, Hkv=2, N=256, d=64, dtype="f16", causal=False,
              seed=0, k_offset_std=2.0, outliers=0, outlier_scale=20.0,
              sparse=None):
    """Inputs of an arbitrary small problem with the same law as the workloads."""
    p = Problem(B, Hq, Hkv, N, d, dtype, causal, sparse, k_offset_std,
                outliers, outlier_scale, f"case B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} {dtype}")
    return p, make_problem_inputs(p, seed)
