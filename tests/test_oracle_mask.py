"""Pins of the oracle's block mask: a hand-worked score, the selection's defining
properties checked by brute force, planted blocks and the degenerate ratios."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.mask import block_scores, select_blocks, valid_blocks, max_keep

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_scores():
    g = json.load(open(os.path.join(GOLDEN, "score_worked_example.json")))
    qc, qs = oracle.pool_vector_quant(np.array([g["q_pool"]], dtype=np.float32))
    kc, ks = oracle.pool_vector_quant(np.array(g["k_pool"], dtype=np.float32))
    assert qc[0].tolist() == g["q_codes"] and float(qs[0]) == g["q_scale"]
    assert kc.tolist() == g["k_codes"] and ks.tolist() == g["k_scale"]
    sc = block_scores(qc, qs, kc, ks)
    assert sc[0].tolist() == g["scores"]
    # the tie between blocks 0 and 3 goes to the lower index: with one slot,
    # non-causal query block 5 of 8 key blocks (forced {0, 10, 11} are outside)
    row = np.full(16, -1e9, dtype=np.float32)
    row[[1, 3, 7]] = [7040.5, 7040.5, 5.0]
    kept, tie = select_blocks(row, 5, 16, False, 1, 16)
    assert kept == [0, 1, 10, 11]
    assert tie


def _brute_force_check(scores, i, nkb, causal, num, den, kept):
    valid = set(valid_blocks(i, nkb, causal))
    forced = {j for j in valid if j == 0 or (64 * j < 128 * i + 128 and 64 * j + 64 > 128 * i)}
    assert set(kept) >= forced
    assert kept == sorted(kept)
    k = -(-len(valid) * num // den)
    rest = valid - forced
    chosen = set(kept) - forced
    assert chosen <= rest
    assert len(chosen) == min(k, len(rest))
    dropped = rest - chosen
    for a in chosen:
        for b in dropped:
            assert (scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("num,den", [(1, 10), (1, 4), (1, 1), (0, 1), (3, 7)])
def test_selection_brute_force(causal, num, den):
    rng = np.random.default_rng(num * 31 + den + causal)
    nkb = 16
    for trial in range(40):
        # coarse values make exact ties common
        scores = rng.integers(-4, 5, nkb).astype(np.float32)
        for i in range(nkb // 2):
            kept, _ = select_blocks(scores, i, nkb, causal, num, den)
            _brute_force_check(scores, i, nkb, causal, num, den, kept)
            if num == den:
                assert kept == valid_blocks(i, nkb, causal)


def test_planted_blocks_are_kept():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, nqb, nkb, d = 1, 4, 2, 8, 16, 64
    qp = rng.standard_normal((B, Hq, nqb, d)).astype(np.float32) * 0.1
    kp = rng.standard_normal((B, Hkv, nkb, d)).astype(np.float32) * 0.1
    planted = {}
    for hq in range(Hq):
        for i in range(2, nqb):
            j = int(rng.integers(1, 2 * i))  # valid, non-forced under causal
            planted[(hq, i)] = j
    # plant one strong block per (kv head): every query block of the group
    # shares the kv head, so plant along a direction shared by its queries
    for hk in range(Hkv):
        direction = rng.standard_normal(d).astype(np.float32)
        for hq in range(hk * 2, hk * 2 + 2):
            qp[0, hq] += direction
        kp[0, hk, 3] += 5 * direction
    idx, cnt, ties = oracle.block_mask(qp, kp, Hq, Hkv, True, 1, 10)
    for hq in range(Hq):
        for i in range(2, nqb):
            kept = idx[0, hq, i, :cnt[0, hq, i]].tolist()
            assert 3 in kept
    assert idx.shape[-1] == max_keep(nkb * 64, 1, 10)


def test_keep_all_and_keep_none():
    rng = np.random.default_rng(2)
    qp = rng.standard_normal((1, 2, 4, 64)).astype(np.float32)
    kp = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    idx, cnt, _ = oracle.block_mask(qp, kp, 2, 1, True, 1, 1)
    for i in range(4):
        assert idx[0, 0, i, :cnt[0, 0, i]].tolist() == list(range(2 * i + 2))
    idx, cnt, _ = oracle.block_mask(qp, kp, 2, 1, True, 0, 1)
    for i in range(4):
        assert idx[0, 1, i, :cnt[0, 1, i]].tolist() == sorted({0, 2 * i, 2 * i + 1})
        assert (idx[0, 1, i, cnt[0, 1, i]:] == -1).all()
    idx, cnt, _ = oracle.block_mask(qp, kp, 2, 1, False, 0, 1)
    assert idx[0, 0, 3, :cnt[0, 0, 3]].tolist() == [0, 6, 7]


def test_max_keep_bound():
    assert max_keep(32768, 1, 10) == 55
    assert max_keep(256, 1, 1) == 4
    assert max_keep(1024, 0, 1) == 3
