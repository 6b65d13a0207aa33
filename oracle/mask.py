"""Block mask from INT8 mean-pooled block scores (oracle; test infrastructure only).

Score: the ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
summary, method, heuristic block selection: the importance of a query block i /
key block j pair is the dot product of the two block mean vectors,
S_hat[i, j] = qbar_i . kbar_j, and the top-k pairs are selected.
Skipping the rest and always keeping the first (sink) and diagonal (local)
blocks follows the SALE explainer (aibr.jp/archives/118208), section 3: a cheap
estimate becomes a block-sparse plan, and weight that concentrates at the start
of a row and near the diagonal gives vertical and slash stripes.

Readings where the pages are silent:

* the pooled vectors are INT8-quantized one vector at a time (same rule as the
  token blocks), the dot product of the codes is exact integer arithmetic, and
  score = fl32(fl32(float32(dot) * q_scale) * k_scale);
* blocks: query block 128 tokens, key block 64 tokens; a key block is valid for
  query block i when (causal) its first key is at or before the block's last
  query, else always;
* forced blocks: key block 0 and the key blocks that overlap the query block's
  token range (2i and 2i+1), when valid;
* k = ceil(|valid| * keep_num / keep_den) in integer arithmetic, taken from the
  valid, non-forced blocks by (score descending, block index ascending);
* the kept list is forced + top, ascending, padded with -1 to max_keep.
"""

from __future__ import annotations

import numpy as np

from .quant import pool_vector_quant, Q_BLOCK, K_BLOCK


def max_keep(N: int, keep_num: int, keep_den: int) -> int:
    """Upper bound on the kept list length of any query block."""
    nkb = N // K_BLOCK
    return min(nkb, 3 + (nkb * keep_num + keep_den - 1) // keep_den)


def block_scores(qp_codes, qp_scale, kp_codes, kp_scale) -> np.ndarray:
    """fp32 scores [nq, nk] of INT8 pooled vectors (exact int dot, two roundings)."""
    dot = qp_codes.astype(np.int64) @ kp_codes.astype(np.int64).T
    dotf = dot.astype(np.float32)   # exact: |dot| <= d * 127^2 < 2^24 for d <= 128
    s1 = dotf * np.asarray(qp_scale, dtype=np.float32)[:, None]
    return s1 * np.asarray(kp_scale, dtype=np.float32)[None, :]


def valid_blocks(i: int, nkb: int, causal: bool):
    if not causal:
        return list(range(nkb))
    last = (Q_BLOCK * i + Q_BLOCK - 1) // K_BLOCK
    return list(range(min(nkb, last + 1)))


def forced_blocks(i: int, valid):
    vs = set(valid)
    lo = (Q_BLOCK * i) // K_BLOCK
    hi = (Q_BLOCK * i + Q_BLOCK - 1) // K_BLOCK
    f = {0} | set(range(lo, hi + 1))
    return sorted(f & vs)


def select_blocks(scores_row: np.ndarray, i: int, nkb: int, causal: bool,
                  keep_num: int, keep_den: int):
    """Kept key blocks of query block i, ascending; plus a near-tie flag.

    The flag is set when the k-th and (k+1)-th ranked candidate scores differ by
    at most 1e-6 relative, i.e. when a different fp32 rounding could have swapped
    them.
    """
    valid = valid_blocks(i, nkb, causal)
    forced = forced_blocks(i, valid)
    k = (len(valid) * keep_num + keep_den - 1) // keep_den
    fset = set(forced)
    rest = [j for j in valid if j not in fset]
    order = sorted(rest, key=lambda j: (-float(scores_row[j]), j))
    take = min(k, len(rest))
    top = order[:take]
    near_tie = False
    if 0 < take < len(order):
        a = float(scores_row[order[take - 1]])
        b = float(scores_row[order[take]])
        near_tie = abs(a - b) <= 1e-6 * max(abs(a), abs(b))
    return sorted(fset | set(top)), near_tie


def block_mask(q_pool, k_pool, Hq: int, Hkv: int, causal: bool,
               keep_num: int, keep_den: int, mk: int | None = None, heads=None):
    """Keep lists for every (batch, query head, query block).

    q_pool [B,Hq,N/128,d] f32, k_pool [B,Hkv,N/64,d] f32.
    Returns (kv_idx int32 [B,Hq,N/128,mk] ascending with -1 padding,
    kv_cnt int32 [B,Hq,N/128], near_tie bool [B,Hq,N/128]).
    ``heads`` optionally restricts the work to a list of (b, hq); other rows
    are left at -1 / 0.
    """
    q_pool = np.asarray(q_pool, dtype=np.float32)
    k_pool = np.asarray(k_pool, dtype=np.float32)
    B, _, nqb, d = q_pool.shape
    nkb = k_pool.shape[2]
    N = nkb * K_BLOCK
    if mk is None:
        mk = max_keep(N, keep_num, keep_den)
    group = Hq // Hkv
    kv_idx = np.full((B, Hq, nqb, mk), -1, dtype=np.int32)
    kv_cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    ties = np.zeros((B, Hq, nqb), dtype=bool)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in heads:
        hk = hq // group
        qc, qs = pool_vector_quant(q_pool[b, hq])
        kc, ks = pool_vector_quant(k_pool[b, hk])
        sc = block_scores(qc, qs, kc, ks)
        for i in range(nqb):
            kept, tie = select_blocks(sc[i], i, nkb, causal, keep_num, keep_den)
            kv_idx[b, hq, i, :len(kept)] = kept
            kv_cnt[b, hq, i] = len(kept)
            ties[b, hq, i] = tie
    return kv_idx, kv_cnt, ties
