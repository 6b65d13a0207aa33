"""Anchor-based stripe selection and attention over gathered keys (oracle;
test infrastructure only).

The AnchorAttention explainer (aibr.jp/archives/118418), section 3: an
approximate maximum score (the anchor) is taken from the initial tokens and a
local window; every other key position is kept when its score comes within a
threshold of the anchor -- a direct comparison, no sort -- which selects
discrete key positions at stripe granularity; the attention then reads those
discrete keys and values instead of contiguous blocks. The page gives no
formulas. Readings:

* a query block (128 rows) shares one stripe set: the score of key k is the
  pooled-mask score of the block's mean query against that single key,
  score(k) = fl32(fl32(dot * sq) * sk[k // 64]) with dot the exact product of
  the INT8 codes of the mean query (quantized on its own, as in
  ``mask.block_scores``) and key k's INT8 code (the smoothed K of
  ``smooth_quant``), sk its block scale;
* the anchor region is the first 64 keys (the initial tokens) and the block's
  own 128 positions (the local window), causally valid ones only; the anchor
  is the largest score there;
* key k (causally valid) is kept when it lies in the anchor region or when
  score(k) >= fl32(anchor - theta); theta is the caller's threshold in score
  units;
* the kept keys, ascending, form the list; a list longer than its capacity
  keeps the anchor region and, of the other kept keys, the lowest indices;
* the attention takes the list 64 entries at a time (the last group may be
  shorter) through the online softmax of ``attention._online_step``, with
  each key's own block scale: s = fl32(S * fl32(alpha_q * sk[k // 64])).
"""

from __future__ import annotations

import numpy as np

from .quant import Q_BLOCK, K_BLOCK, pool_vector_quant
from .attention import softmax_scale_log2, _online_step, _finish, _dtypes
from .rounding import round_to_dtype

GATHER_TILE = 64


def stripe_scores(q_pool, k_i8, k_scale, Hq: int, Hkv: int):
    """Scores [B, Hq, N/128, N] f32 of each query block's mean query against
    every single key."""
    q_pool = np.asarray(q_pool, dtype=np.float32)
    B, _, nqb, d = q_pool.shape
    N = k_i8.shape[2]
    group = Hq // Hkv
    out = np.zeros((B, Hq, nqb, N), dtype=np.float32)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // group
            qc, qs = pool_vector_quant(q_pool[b, hq])            # [nqb, d], [nqb]
            dot = qc.astype(np.int64) @ k_i8[b, hk].astype(np.int64).T   # exact
            s1 = (dot.astype(np.float32) * np.asarray(qs, np.float32)[:, None]).astype(np.float32)
            sk = np.asarray(k_scale[b, hk], np.float32)[np.arange(N) // K_BLOCK]
            out[b, hq] = (s1 * sk[None, :]).astype(np.float32)
    return out


def anchor_region(i: int, N: int, causal: bool):
    """Initial tokens and local window of query block i (causally valid)."""
    last = Q_BLOCK * i + Q_BLOCK - 1 if causal else N - 1
    keys = set(range(min(K_BLOCK, N))) | set(range(Q_BLOCK * i, Q_BLOCK * i + Q_BLOCK))
    return sorted(k for k in keys if k <= last)


def stripe_select(q_pool, k_i8, k_scale, Hq: int, Hkv: int, causal: bool, theta: float,
                  max_keys: int):
    """Kept key lists [B, Hq, N/128, max_keys] int32 (ascending, -1 padded),
    counts [B, Hq, N/128] int32, and the scores."""
    sc = stripe_scores(q_pool, k_i8, k_scale, Hq, Hkv)
    B, _, nqb, N = sc.shape
    idx = np.full((B, Hq, nqb, max_keys), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    th = np.float32(theta)
    for b in range(B):
        for h in range(Hq):
            for i in range(nqb):
                s = sc[b, h, i]
                nvis = min(N, Q_BLOCK * i + Q_BLOCK) if causal else N
                region = anchor_region(i, N, causal)
                anchor = np.float32(max(s[k] for k in region))
                thr = np.float32(anchor - th)
                rset = set(region)
                others = [k for k in range(nvis) if k not in rset and s[k] >= thr]
                room = max(0, max_keys - len(region))
                kept = sorted(region + others[:room])[:max_keys]
                idx[b, h, i, :len(kept)] = kept
                cnt[b, h, i] = len(kept)
    return idx, cnt, sc


def emulate_stripe_attention(q_i8, q_scale, k_i8, k_scale, v, causal: bool, Hq: int, Hkv: int,
                             key_idx, key_cnt, p_dtype: str | None = None,
                             out_dtype: str | None = None, blocks=None, tau: float = 0.0):
    """The quantized path over gathered keys, 64 list entries per online step.
    Returns (O, O_pre, lse) as ``attention.emulate_attention``."""
    p_dtype, out_dtype = _dtypes(v, p_dtype, out_dtype)
    from .quant import _as_f64
    v64 = _as_f64(v)
    B, _, N, d = q_i8.shape
    group = Hq // Hkv
    c = softmax_scale_log2(d)
    nqb = N // Q_BLOCK
    O = np.full((B, Hq, N, d), np.nan, dtype=np.float32)
    O_pre = np.full((B, Hq, N, d), np.nan, dtype=np.float32)
    lse = np.full((B, Hq, N), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nqb)]
    ninf = np.float32(-np.inf)
    for b, hq, i in blocks:
        hk = hq // group
        r0 = i * Q_BLOCK
        rows = np.arange(r0, r0 + Q_BLOCK)
        qc = q_i8[b, hq, r0:r0 + Q_BLOCK].astype(np.float64)
        alpha_q = np.float32(np.float32(q_scale[b, hq, i]) * c)
        m = np.full(Q_BLOCK, ninf, dtype=np.float32)
        l = np.zeros(Q_BLOCK)
        acc = np.zeros((Q_BLOCK, d))
        keys_all = np.asarray(key_idx[b, hq, i, :key_cnt[b, hq, i]], dtype=np.int64)
        for t0 in range(0, len(keys_all), GATHER_TILE):
            keys = keys_all[t0:t0 + GATHER_TILE]
            S = qc @ k_i8[b, hk, keys].astype(np.float64).T
            alpha = (alpha_q * np.asarray(k_scale[b, hk, keys // K_BLOCK], np.float32)
                     ).astype(np.float32)
            s = (S.astype(np.float32) * alpha[None, :]).astype(np.float32)
            if causal:
                s = np.where(keys[None, :] <= rows[:, None], s, ninf)
            m, l, acc = _online_step(m, l, acc, s, v64[b, hk, keys], p_dtype, tau)
        o32, lse[b, hq, r0:r0 + Q_BLOCK] = _finish(m, l, acc)
        O_pre[b, hq, r0:r0 + Q_BLOCK] = o32
        O[b, hq, r0:r0 + Q_BLOCK] = round_to_dtype(o32, out_dtype)
    return O, O_pre, lse
