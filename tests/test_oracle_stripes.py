"""Pins of the anchor-based stripe selection and the gathered-key emulation
(oracle/stripes.py).

* the scores against a scalar brute force (exact integer dot, two fp32
  roundings);
* the selection against its definition, brute-forced per key: anchor region
  always kept, others kept iff score >= fl32(anchor - theta), capacity rule;
* theta = +inf keeps every visible key, and the gathered emulation is then the
  dense INT8 emulation bit for bit; lists made of whole aligned 64-key blocks
  give the block-sparse emulation bit for bit;
* V = 1 gives 1 within V's unit roundoff; the emulation is close to exact
  attention over the same keys.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import emulate_attention
from oracle.quant import pool_vector_quant
from oracle.stripes import (anchor_region, emulate_stripe_attention, stripe_scores,
                            stripe_select)
from synthetic import make_case


def _sq(p, t):
    return oracle.smooth_quant(t["q"], t["k"], pools=True)


def test_scores_brute_force():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype="bf16", causal=True, seed=91,
                     k_offset_std=3.0)
    sq = _sq(p, t)
    sc = stripe_scores(sq["q_pool"], sq["k_i8"], sq["k_scale"], 2, 1)
    for h in range(2):
        qc, qs = pool_vector_quant(sq["q_pool"][0, h])
        for i in range(2):
            for k in range(0, 256, 7):
                dot = sum(int(qc[i, x]) * int(sq["k_i8"][0, 0, k, x]) for x in range(64))
                want = np.float32(np.float32(np.float32(dot) * np.float32(qs[i]))
                                  * np.float32(sq["k_scale"][0, 0, k // 64]))
                assert sc[0, h, i, k] == want


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("theta", [0.0, 0.5, 2.0])
def test_selection_definition(causal, theta):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=causal, seed=92,
                     k_offset_std=2.0)
    sq = _sq(p, t)
    idx, cnt, sc = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 2, 1, causal, theta,
                                 512)
    for h in range(2):
        for i in range(4):
            nvis = 128 * i + 128 if causal else 512
            region = anchor_region(i, 512, causal)
            anchor = max(float(sc[0, h, i, k]) for k in region)
            thr = float(np.float32(np.float32(anchor) - np.float32(theta)))
            want = [k for k in range(nvis) if k in region or float(sc[0, h, i, k]) >= thr]
            assert list(idx[0, h, i, :cnt[0, h, i]]) == want
            assert all(x == -1 for x in idx[0, h, i, cnt[0, h, i]:])


def test_capacity_keeps_the_anchor_region_and_the_lowest_others():
    p, t = make_case(B=1, Hq=1, Hkv=1, N=1024, d=64, dtype="bf16", causal=True, seed=93)
    sq = _sq(p, t)
    full, fcnt, _ = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 1, 1, True, 1e30, 1024)
    idx, cnt, _ = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 1, 1, True, 1e30, 256)
    i = 7
    region = anchor_region(i, 1024, True)
    others = [k for k in full[0, 0, i, :fcnt[0, 0, i]] if k not in set(region)]
    want = sorted(region + others[:256 - len(region)])
    assert list(idx[0, 0, i, :cnt[0, 0, i]]) == want


def test_theta_inf_is_the_dense_emulation():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=94,
                     k_offset_std=3.0)
    sq = _sq(p, t)
    idx, cnt, _ = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 2, 1, True, 1e30, 512)
    for i in range(4):
        assert list(idx[0, 0, i, :cnt[0, 0, i]]) == list(range(128 * i + 128))
    a = emulate_stripe_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
                                 True, 2, 1, idx, cnt, tau=8.0)
    b = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 2,
                          1, tau=8.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_whole_block_lists_are_the_block_sparse_emulation():
    p, t = make_case(B=1, Hq=1, Hkv=1, N=768, d=128, dtype="f16", causal=False, seed=95)
    sq = _sq(p, t)
    blocks = [0, 3, 5, 11]
    keys = np.concatenate([np.arange(64 * j, 64 * j + 64) for j in blocks])
    idx = np.tile(keys.astype(np.int32), (1, 1, 6, 1))
    cnt = np.full((1, 1, 6), len(keys), dtype=np.int32)
    kv_idx = np.tile(np.array(blocks, np.int32), (1, 1, 6, 1))
    kv_cnt = np.full((1, 1, 6), len(blocks), dtype=np.int32)
    a = emulate_stripe_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
                                 False, 1, 1, idx, cnt, tau=8.0)
    b = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], False, 1,
                          1, kv_idx=kv_idx, kv_cnt=kv_cnt, tau=8.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_v_ones_and_closeness_to_exact(dtype):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype=dtype, causal=True, seed=96,
                     k_offset_std=2.0)
    sq = _sq(p, t)
    idx, cnt, _ = stripe_select(sq["q_pool"], sq["k_i8"], sq["k_scale"], 2, 1, True, 1.0, 512)
    ones = torch.ones_like(t["v"])
    O, Opre, _ = emulate_stripe_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                          ones, True, 2, 1, idx, cnt, tau=8.0)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.abs(Opre - 1).max() <= u * (1 + 1e-6) and np.abs(O - 1).max() <= u
    _, Opre, _ = emulate_stripe_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                          t["v"], True, 2, 1, idx, cnt, tau=8.0)
    q, k, v = (t[x].double().numpy()[0] for x in "qkv")
    num = den = 0.0
    for h in range(2):
        for i in range(4):
            keys = idx[0, h, i, :cnt[0, h, i]]
            for r in range(128 * i, 128 * i + 128):
                kk = keys[keys <= r]
                s = q[h, r] @ k[0, kk].T / math.sqrt(64)
                w = np.exp(s - s.max())
                ex = (w @ v[0, kk]) / w.sum()
                num += float(ex @ Opre[0, h, r])
                den += math.sqrt(float(ex @ ex) * float(Opre[0, h, r] @ Opre[0, h, r]))
    assert num / den > 0.999
