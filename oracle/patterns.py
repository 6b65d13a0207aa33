"""Vertical and slash pattern prediction on top of a block plan (oracle; test
infrastructure only).

The SALE explainer (aibr.jp/archives/118208), sections 1 and 3: besides the
element-level 4-bit estimates, the method uses the statistical tendencies of
the attention map to predict vertical lines (key positions that matter to
every query) and slash lines (a fixed distance between query and key). The
page gives no rule. Readings taken here:

* the statistics are votes of the per-query-block selections: query block i
  votes for every key block j of its kept set that is not forced (the sink
  block 0 and the diagonal blocks 2i, 2i+1 are in every plan by rule, so they
  carry no information); a vote counts once for key block j (vertical) and
  once for the offset o = 2i - j (slash: the distance from the query block's
  first diagonal key block, negative past the diagonal when not causal);
* a kept set is the set of the list's entries that are valid key blocks for
  the query block (0 <= j < N/64, and j <= 2i + 1 when causal): duplicates and
  invalid entries count once or not at all;
* the predicted lines of a (batch, query head) are the n_vertical key blocks
  and the n_slash offsets with the most votes, at least two each (one query
  block's choice is not a tendency), ties to the lower key block, or to the
  lower offset (the nearer one to the diagonal when causal);
* every query block then keeps, on top of its own set, the predicted vertical
  blocks and the blocks 2i - o of the predicted offsets that are valid for it;
  the output lists are ascending.
"""

from __future__ import annotations

import numpy as np

from .quant import Q_BLOCK, K_BLOCK

MAX_LINES = 64          # most vertical or slash lines per head
NO_SLASH = np.iinfo(np.int32).min


def _valid(j: int, i: int, nkb: int, causal: bool) -> bool:
    if j < 0 or j >= nkb:
        return False
    return not causal or K_BLOCK * j <= Q_BLOCK * i + Q_BLOCK - 1


def _forced(i: int, nkb: int, causal: bool) -> set:
    lo = (Q_BLOCK * i) // K_BLOCK
    hi = (Q_BLOCK * i + Q_BLOCK - 1) // K_BLOCK
    return {j for j in {0} | set(range(lo, hi + 1)) if _valid(j, i, nkb, causal)}


def kept_set(row, cnt: int, i: int, nkb: int, causal: bool) -> set:
    """The valid key blocks among the first cnt entries of a kept list."""
    return {int(j) for j in np.asarray(row)[:max(0, cnt)] if _valid(int(j), i, nkb, causal)}


def pattern_votes(kv_idx, kv_cnt, N: int, causal: bool):
    """Vertical votes [B, Hq, N/64] and slash votes [B, Hq, 2*N/64 - 1] (offset o
    at index o + N/64 - 1) of the non-forced kept blocks of every query block."""
    kv_idx = np.asarray(kv_idx)
    kv_cnt = np.asarray(kv_cnt)
    B, Hq, nqb, mk = kv_idx.shape
    nkb = N // K_BLOCK
    vert = np.zeros((B, Hq, nkb), dtype=np.int64)
    slash = np.zeros((B, Hq, 2 * nkb - 1), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            for i in range(nqb):
                ks = kept_set(kv_idx[b, h, i], min(int(kv_cnt[b, h, i]), mk), i, nkb, causal)
                for j in ks - _forced(i, nkb, causal):
                    vert[b, h, j] += 1
                    slash[b, h, 2 * i - j + nkb - 1] += 1
    return vert, slash


def top_lines(votes: np.ndarray, n: int) -> list:
    """Indices of the n largest vote counts of at least 2, ties to the lower
    index, in rank order."""
    cand = [(-int(v), x) for x, v in enumerate(votes) if v >= 2]
    cand.sort()
    return [x for _, x in cand[:n]]


def predict_patterns(kv_idx, kv_cnt, N: int, causal: bool, n_vertical: int, n_slash: int,
                     mk_out: int | None = None):
    """Extend every kept list with the predicted vertical and slash blocks.

    kv_idx [B, Hq, N/128, mk] int32, kv_cnt [B, Hq, N/128] (counts above mk
    read mk entries). Returns (lines [B, Hq, n_vertical + n_slash] int32: the
    vertical key blocks in rank order padded with -1, then the slash offsets
    in rank order padded with INT32_MIN; kv_idx_out [B, Hq, N/128, mk_out]
    ascending with -1 padding; kv_cnt_out [B, Hq, N/128]).
    """
    kv_idx = np.asarray(kv_idx)
    kv_cnt = np.asarray(kv_cnt)
    B, Hq, nqb, mk = kv_idx.shape
    nkb = N // K_BLOCK
    if mk_out is None:
        mk_out = min(nkb, mk + n_vertical + n_slash)
    vert, slash = pattern_votes(kv_idx, kv_cnt, N, causal)
    lines = np.empty((B, Hq, n_vertical + n_slash), dtype=np.int32)
    out_idx = np.full((B, Hq, nqb, mk_out), -1, dtype=np.int32)
    out_cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            vsel = top_lines(vert[b, h], n_vertical)
            ssel = [x - (nkb - 1) for x in top_lines(slash[b, h], n_slash)]
            lines[b, h, :n_vertical] = vsel + [-1] * (n_vertical - len(vsel))
            lines[b, h, n_vertical:] = ssel + [NO_SLASH] * (n_slash - len(ssel))
            for i in range(nqb):
                ks = kept_set(kv_idx[b, h, i], min(int(kv_cnt[b, h, i]), mk), i, nkb, causal)
                ks |= {j for j in vsel if _valid(j, i, nkb, causal)}
                ks |= {2 * i - o for o in ssel if _valid(2 * i - o, i, nkb, causal)}
                row = sorted(ks)
                assert len(row) <= mk_out
                out_idx[b, h, i, :len(row)] = row
                out_cnt[b, h, i] = len(row)
    return lines, out_idx, out_cnt
