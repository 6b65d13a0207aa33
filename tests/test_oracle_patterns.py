"""Pins of the vertical / slash pattern prediction (oracle.patterns).

* A hand-worked causal example (four query blocks, eight key blocks): the
  votes, the predicted lines and the extended lists, worked out by hand from
  the rule and written here as literals.
* A hand-worked non-causal example with a slash past the diagonal (negative
  offset).
* No lines asked for: the output is each list's valid entries, ascending,
  once each.
* Planted lines: a key block kept by most query blocks (a vertical line) and a
  fixed distance kept by most (a slash line) reach every query block that can
  see them, and nothing else is added.
* Invariants: every input block stays, every added block lies on a predicted
  line, the vote totals equal the number of non-forced kept blocks.
"""

import numpy as np
import pytest

from oracle.patterns import predict_patterns, pattern_votes, NO_SLASH


def _lists(rows, mk):
    nqb = len(rows)
    idx = np.full((1, 1, nqb, mk), -1, dtype=np.int32)
    cnt = np.zeros((1, 1, nqb), dtype=np.int32)
    for i, r in enumerate(rows):
        idx[0, 0, i, :len(r)] = r
        cnt[0, 0, i] = len(r)
    return idx, cnt


# N = 512: query blocks 0..3 (128 rows), key blocks 0..7 (64 keys). Causal:
# block i sees key blocks 0..2i+1; forced are 0, 2i and 2i+1.
HAND_ROWS = [[0, 1], [0, 1, 2, 3], [0, 1, 3, 4, 5], [0, 3, 5, 6, 7, 7, 9]]


def test_hand_worked_votes():
    idx, cnt = _lists(HAND_ROWS, 7)
    vert, slash = pattern_votes(idx, cnt, 512, True)
    # row 1 votes {1}; row 2 votes {1, 3}; row 3 votes {3, 5} (7 is forced and
    # repeated, 9 is no key block)
    assert vert[0, 0].tolist() == [0, 2, 0, 2, 0, 1, 0, 0]
    # offsets 2i - j: row 1: 1; row 2: 3, 1; row 3: 3, 1  (index o + 7)
    want = [0] * 15
    want[1 + 7], want[3 + 7] = 3, 2
    assert slash[0, 0].tolist() == want


def test_hand_worked_one_line_each():
    idx, cnt = _lists(HAND_ROWS, 7)
    lines, oi, oc = predict_patterns(idx, cnt, 512, True, 1, 1)
    # vertical: blocks 1 and 3 tie at two votes -> block 1; slash: offset 1
    assert lines[0, 0].tolist() == [1, 1]
    want = [[0, 1], [0, 1, 2, 3], [0, 1, 3, 4, 5], [0, 1, 3, 5, 6, 7]]
    assert oc[0, 0].tolist() == [len(r) for r in want]
    for i, r in enumerate(want):
        assert oi[0, 0, i].tolist() == r + [-1] * (oi.shape[-1] - len(r))


def test_hand_worked_more_lines_than_tendencies():
    idx, cnt = _lists(HAND_ROWS, 7)
    lines, oi, oc = predict_patterns(idx, cnt, 512, True, 3, 3)
    # block 5 has one vote only; offsets 1 and 3 qualify
    assert lines[0, 0].tolist() == [1, 3, -1, 1, 3, NO_SLASH]
    want = [[0, 1], [0, 1, 2, 3], [0, 1, 3, 4, 5], [0, 1, 3, 5, 6, 7]]
    for i, r in enumerate(want):
        assert oi[0, 0, i, :oc[0, 0, i]].tolist() == r


def test_hand_worked_non_causal_negative_offset():
    # N = 384, not causal: query blocks 0..2 see key blocks 0..5; forced 0, 2i, 2i+1
    rows = [[0, 1, 4], [0, 2, 3, 5], [0, 4, 5, 1]]
    idx, cnt = _lists(rows, 4)
    vert, slash = pattern_votes(idx, cnt, 384, False)
    # votes: row 0: 4 (offset -4); row 1: 5 (offset -3); row 2: 1 (offset 3)
    assert vert[0, 0].tolist() == [0, 1, 0, 0, 1, 1]
    lines, oi, oc = predict_patterns(idx, cnt, 384, False, 2, 2)
    assert lines[0, 0].tolist() == [-1, -1, NO_SLASH, NO_SLASH]   # no line has two votes
    rows2 = [[0, 1, 3], [0, 2, 3, 5], [0, 4, 5, 3, 1]]
    idx, cnt = _lists(rows2, 5)
    # row 0 votes 3 (offset -3); row 1 votes 5 (offset -3); row 2 votes 3, 1
    # (offsets 1, 3): vertical 3 has two votes, offset -3 has two
    lines, oi, oc = predict_patterns(idx, cnt, 384, False, 1, 1)
    assert lines[0, 0].tolist() == [3, -3]
    # row 0 gains 0 - (-3) = 3 (already there); row 1 gains 3 and 2 + 3 = 5;
    # row 2 gains 3 and 4 + 3 = 7 (no key block)
    want = [[0, 1, 3], [0, 2, 3, 5], [0, 1, 3, 4, 5]]
    for i, r in enumerate(want):
        assert oi[0, 0, i, :oc[0, 0, i]].tolist() == r


def test_no_lines_is_the_valid_set():
    rng = np.random.default_rng(3)
    nqb, nkb, mk = 8, 16, 9
    idx = rng.integers(-3, nkb + 3, (2, 3, nqb, mk)).astype(np.int32)
    cnt = rng.integers(0, mk + 4, (2, 3, nqb)).astype(np.int32)
    for causal in (True, False):
        lines, oi, oc = predict_patterns(idx, cnt, nkb * 64, causal, 0, 0)
        assert lines.shape == (2, 3, 0)
        for b in range(2):
            for h in range(3):
                for i in range(nqb):
                    ents = idx[b, h, i, :min(cnt[b, h, i], mk)]
                    ok = sorted({int(j) for j in ents if 0 <= j < nkb
                                 and (not causal or j <= 2 * i + 1)})
                    assert oi[b, h, i, :oc[b, h, i]].tolist() == ok
                    assert np.all(oi[b, h, i, oc[b, h, i]:] == -1)


@pytest.mark.parametrize("causal", [True, False])
def test_planted_lines_reach_every_query_block(causal):
    rng = np.random.default_rng(5)
    nqb, nkb = 16, 32
    N = nkb * 64
    rows = []
    for i in range(nqb):
        vis = 2 * i + 2 if causal else nkb
        r = {0, 2 * i, 2 * i + 1} & set(range(vis))
        # background: one random block per row (at most one vote per block)
        r.add(int(rng.integers(0, vis)))
        # vertical line at key block 6 in most rows that see it
        if vis > 6 and i % 5 != 0:
            r.add(6)
        # slash line at distance 3 behind the diagonal in most rows
        if 2 * i - 3 >= 0 and i % 4 != 1:
            r.add(2 * i - 3)
        rows.append(sorted(r))
    idx, cnt = _lists(rows, max(len(r) for r in rows))
    lines, oi, oc = predict_patterns(idx, cnt, N, causal, 1, 1)
    assert lines[0, 0].tolist() == [6, 3]
    for i in range(nqb):
        got = set(oi[0, 0, i, :oc[0, 0, i]].tolist())
        vis = 2 * i + 2 if causal else nkb
        want = set(rows[i])
        if vis > 6:
            want.add(6)
        if 0 <= 2 * i - 3 < vis:
            want.add(2 * i - 3)
        assert got == want


def test_invariants_on_random_lists():
    rng = np.random.default_rng(11)
    nqb, nkb, mk = 32, 64, 12
    N = nkb * 64
    for causal in (True, False):
        idx = rng.integers(-1, nkb + 1, (1, 2, nqb, mk)).astype(np.int32)
        cnt = rng.integers(0, mk + 1, (1, 2, nqb)).astype(np.int32)
        nv, ns = 5, 4
        vert, slash = pattern_votes(idx, cnt, N, causal)
        lines, oi, oc = predict_patterns(idx, cnt, N, causal, nv, ns)
        for h in range(2):
            nonforced = 0
            vl = [int(x) for x in lines[0, h, :nv] if x >= 0]
            sl = [int(x) for x in lines[0, h, nv:] if x != NO_SLASH]
            for i in range(nqb):
                vis = 2 * i + 2 if causal else nkb
                kept = {int(j) for j in idx[0, h, i, :cnt[0, h, i]] if 0 <= j < min(vis, nkb)}
                nonforced += len(kept - {0, 2 * i, 2 * i + 1})
                got = set(oi[0, h, i, :oc[0, h, i]].tolist())
                assert kept <= got
                for j in got - kept:
                    assert j in vl or (2 * i - j) in sl
                assert oi[0, h, i, :oc[0, h, i]].tolist() == sorted(got)
            assert vert[0, h].sum() == nonforced == slash[0, h].sum()
            # lines in rank order: votes non-increasing, at least 2
            vv = [int(vert[0, h, j]) for j in vl]
            assert vv == sorted(vv, reverse=True) and all(v >= 2 for v in vv)
