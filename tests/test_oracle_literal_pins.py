"""Literal pins of two oracle definitions that the other CPU tests only use
(their expected answers would otherwise come from the same functions):

* the anchor region of the stripe selection (AnchorAttention explainer,
  aibr.jp/archives/118418, section 3: the anchor is taken over the initial
  tokens and a local window). Reading: the first 64 keys and the query
  block's own 128 positions, causally valid ones. The expected key sets below
  are written out by hand.
* the (query row, key) sample of the per-head error proxy (adaptive
  precision, SageAttention explainer, sections 1-4): one row per evenly
  spaced query block at offset (37u + 11) mod 128, one key per evenly spaced
  key block at offset (29w + 5) mod 64. The expected positions are literals
  (worked by hand for a few entries: u = 1 -> 128 + 48 = 176,
  u = 63 -> 8064 + 38 = 8102, w = 127 -> 8128 + 40 = 8168).
"""

import numpy as np
import pytest

import oracle
from oracle.stripes import anchor_region, stripe_select
from oracle.attention import head_error_sample
from synthetic import make_case


def _r(a, b):
    return list(range(a, b))


@pytest.mark.parametrize("N,i,causal,want", [
    (1024, 3, True, _r(0, 64) + _r(384, 512)),
    (1024, 0, True, _r(0, 128)),                 # the window covers the initial tokens
    (1024, 1, True, _r(0, 64) + _r(128, 256)),
    (1024, 7, True, _r(0, 64) + _r(896, 1024)),  # the last block
    (768, 5, False, _r(0, 64) + _r(640, 768)),
    (768, 0, False, _r(0, 128)),
    (128, 0, True, _r(0, 128)),                  # one query block
])
def test_anchor_region_literal(N, i, causal, want):
    assert anchor_region(i, N, causal) == want


def test_anchor_region_is_what_the_selection_keeps_at_minus_infinity():
    # theta = -inf keeps no key outside the region: every list is exactly the
    # hand-written region of its block
    p, t = make_case(B=1, Hq=2, Hkv=1, N=1024, d=64, dtype="bf16", causal=True, seed=5,
                     k_offset_std=2.0)
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, _ = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 2, 1, True,
                                -np.inf, 256)
    for i in range(8):
        want = _r(0, 128) if i == 0 else _r(0, 64) + _r(128 * i, 128 * i + 128)
        for h in range(2):
            assert cnt[0, h, i] == len(want)
            assert idx[0, h, i, :cnt[0, h, i]].tolist() == want


ROWS_8192 = [11, 176, 341, 506, 543, 708, 873, 910, 1075, 1240, 1405, 1442, 1607, 1772, 1809,
             1974, 2139, 2176, 2341, 2506, 2671, 2708, 2873, 3038, 3075, 3240, 3405, 3570, 3607,
             3772, 3937, 3974, 4139, 4304, 4469, 4506, 4671, 4836, 4873, 5038, 5203, 5368, 5405,
             5570, 5735, 5772, 5937, 6102, 6267, 6304, 6469, 6634, 6671, 6836, 7001, 7166, 7203,
             7368, 7533, 7570, 7735, 7900, 7937, 8102]
KEYS_8192 = [5, 98, 191, 220, 313, 342, 435, 464, 557, 586, 679, 708, 801, 894, 923, 1016, 1045,
             1138, 1167, 1260, 1289, 1382, 1411, 1504, 1597, 1626, 1719, 1748, 1841, 1870, 1963,
             1992, 2085, 2114, 2207, 2300, 2329, 2422, 2451, 2544, 2573, 2666, 2695, 2788, 2817,
             2910, 3003, 3032, 3125, 3154, 3247, 3276, 3369, 3398, 3491, 3520, 3613, 3706, 3735,
             3828, 3857, 3950, 3979, 4072, 4101, 4194, 4287, 4316, 4409, 4438, 4531, 4560, 4653,
             4682, 4775, 4804, 4897, 4990, 5019, 5112, 5141, 5234, 5263, 5356, 5385, 5478, 5507,
             5600, 5693, 5722, 5815, 5844, 5937, 5966, 6059, 6088, 6181, 6210, 6303, 6396, 6425,
             6518, 6547, 6640, 6669, 6762, 6791, 6884, 6913, 7006, 7099, 7128, 7221, 7250, 7343,
             7372, 7465, 7494, 7587, 7616, 7709, 7802, 7831, 7924, 7953, 8046, 8075, 8168]


def test_head_error_sample_literal_8192():
    rows, keys = head_error_sample(8192)
    assert rows.tolist() == ROWS_8192
    assert keys.tolist() == KEYS_8192


def test_head_error_sample_literal_small_and_long():
    # N = 1024: fewer blocks than the sample's 64 rows / 256 keys, one per block
    rows, keys = head_error_sample(1024)
    assert rows.tolist() == [11, 176, 341, 506, 543, 708, 873, 910]
    assert keys.tolist() == [5, 98, 191, 220, 313, 342, 435, 464, 557, 586, 679, 708, 801, 894,
                             923, 1016]
    # N = 65536: every 8th query block, every 4th key block
    rows, keys = head_error_sample(65536)
    assert len(rows) == 64 and len(keys) == 256
    assert rows[:6].tolist() == [11, 1072, 2133, 3194, 4127, 5188]
    assert keys[:6].tolist() == [5, 290, 575, 796, 1081, 1302]
