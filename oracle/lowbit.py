"""Element-level low-bit block estimator (oracle; test infrastructure only).

The SALE explainer (aibr.jp/archives/118208), sections 2 and 3: instead of
scoring a (query block, key block) pair by representative vectors, estimate
every query-key product cheaply with 4-bit quantized Q and K, build the
block-sparse plan from those element-level estimates, and keep the sink and
local (vertical and slash) patterns. The page fixes neither the 4-bit format
nor how the estimates become a block score. Readings:

* the 4-bit format is OCP MX FP4: E2M1 elements (magnitudes 0, 0.5, 1, 1.5,
  2, 3, 4, 6) sharing one E8M0 power-of-two scale per 32 consecutive channels
  (the format the CDNA4 matrix cores take). Per the MX v1.0 definition the
  shared exponent is floor(log2(amax)) - 2 (2 is the largest E2M1 exponent),
  each element is x / 2^E rounded to nearest-even on the E2M1 grid and
  saturated at 6; an all-zero block has exponent -127;
* the quantized inputs are the raw Q and the smoothed K (fl32(K) - k_mean, as
  for the INT8 path);
* the estimate of a pair is the exact dot product of the dequantized vectors;
* a block's score is the largest estimate over its causally visible
  (query, key) pairs (an element-level max, where the pooled score of the
  SageAttention-style mask uses block means);
* the kept set is chosen from these scores by the same rule as
  ``mask.select_blocks``: forced first and diagonal blocks (the sink and local
  patterns) plus the top fraction of the rest.
"""

from __future__ import annotations

import math

import numpy as np

from .quant import Q_BLOCK, K_BLOCK, _as_f64, k_channel_mean
from .mask import max_keep, select_blocks

MX_BLOCK = 32
FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def fp4_round(y: np.ndarray) -> np.ndarray:
    """Round to nearest on the E2M1 grid, ties to the even encoding (the grid
    points 0, 1, 2, 4 have an even last bit), saturating at +-6."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 6.0)
    out = np.empty_like(a)
    flat_a, flat_o = a.ravel(), out.ravel()
    for n, v in enumerate(flat_a):
        hi = int(np.searchsorted(FP4_GRID, v, side="left"))
        if hi < len(FP4_GRID) and FP4_GRID[hi] == v:
            flat_o[n] = v
            continue
        lo = hi - 1
        dl, dh = v - FP4_GRID[lo], FP4_GRID[hi] - v
        if dl < dh:
            flat_o[n] = FP4_GRID[lo]
        elif dh < dl:
            flat_o[n] = FP4_GRID[hi]
        else:  # tie: the even encoding (grid index even)
            flat_o[n] = FP4_GRID[lo] if lo % 2 == 0 else FP4_GRID[hi]
    return np.sign(y) * out


def mxfp4_quantize(x: np.ndarray):
    """MX FP4 along the last axis (a multiple of 32).

    Returns (element values on the E2M1 grid [..., d], shared exponents
    [..., d/32] int). The dequantized tensor is values * 2^exponent.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.abs(g).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    vals = fp4_round(g / np.exp2(e.astype(np.float64))[..., None])
    return vals.reshape(x.shape), e


def mxfp4_dequantize(vals, exps):
    d = vals.shape[-1]
    g = vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    return (g * np.exp2(exps.astype(np.float64))[..., None]).reshape(vals.shape)


def lowbit_inputs(q, k, k_mean=None):
    """The dequantized 4-bit Q and smoothed K: ([B,Hq,N,d], [B,Hkv,N,d]) fp64."""
    q64, k64 = _as_f64(q), _as_f64(k)
    m = k_channel_mean(k64) if k_mean is None else np.asarray(k_mean, dtype=np.float32)
    ks32 = k64.astype(np.float32) - m[:, :, None, :]
    qv, qe = mxfp4_quantize(q64.astype(np.float32))
    kv, ke = mxfp4_quantize(ks32)
    return mxfp4_dequantize(qv, qe), mxfp4_dequantize(kv, ke)


def lowbit_scores(q, k, Hq: int, Hkv: int, causal: bool, k_mean=None, heads=None):
    """Block scores [B, Hq, N/128, N/64] (fp64; -inf for causally invalid blocks):
    the largest element-level 4-bit estimate over each block's visible pairs."""
    qd, kd = lowbit_inputs(q, k, k_mean)
    B, _, N, _ = qd.shape
    group = Hq // Hkv
    nqb, nkb = N // Q_BLOCK, N // K_BLOCK
    sc = np.full((B, Hq, nqb, nkb), -np.inf)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    keys = np.arange(N)
    for b, hq in heads:
        hk = hq // group
        for i in range(nqb):
            rows = np.arange(Q_BLOCK * i, Q_BLOCK * i + Q_BLOCK)
            est = qd[b, hq, rows] @ kd[b, hk].T          # [128, N]
            if causal:
                est = np.where(keys[None, :] <= rows[:, None], est, -np.inf)
            blk = est.reshape(Q_BLOCK, nkb, K_BLOCK).max(axis=(0, 2))
            sc[b, hq, i] = blk
    return sc


def lowbit_block_mask(q, k, Hq: int, Hkv: int, causal: bool, keep_num: int, keep_den: int,
                      mk: int | None = None, k_mean=None, heads=None):
    """Kept lists from the element-level 4-bit scores, with the selection rule
    of the pooled mask. Returns (kv_idx, kv_cnt, near_tie, scores)."""
    sc = lowbit_scores(q, k, Hq, Hkv, causal, k_mean, heads)
    B, _, nqb, nkb = sc.shape
    N = nkb * K_BLOCK
    if mk is None:
        mk = max_keep(N, keep_num, keep_den)
    kv_idx = np.full((B, Hq, nqb, mk), -1, dtype=np.int32)
    kv_cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    ties = np.zeros((B, Hq, nqb), dtype=bool)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in heads:
        for i in range(nqb):
            kept, tie = select_blocks(sc[b, hq, i], i, nkb, causal, keep_num, keep_den)
            kv_idx[b, hq, i, :len(kept)] = kept
            kv_cnt[b, hq, i] = len(kept)
            ties[b, hq, i] = tie
    return kv_idx, kv_cnt, ties, sc
