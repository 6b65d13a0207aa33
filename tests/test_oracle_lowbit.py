"""Pins of the element-level 4-bit block estimator (oracle/lowbit.py).

* E2M1 rounding against hand-worked values (every tie, saturation, sign);
* MX FP4 quantization: the shared exponent rule, grid values quantize to
  themselves, the error bound, zero blocks;
* the block score is the max of the dequantized dot products over the
  visible pairs: brute force on a tiny case;
* inputs already on the MX grid make the estimates exact, so the scores are
  the exact block maxima of q . (k - k_mean);
* a planted large element wins its block; keep-all and keep-none.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.lowbit import (FP4_GRID, fp4_round, lowbit_block_mask, lowbit_inputs,
                           lowbit_scores, mxfp4_dequantize, mxfp4_quantize)
from synthetic import make_case


def test_fp4_round_hand_worked():
    cases = {0.0: 0.0, 0.2: 0.0, 0.25: 0.0, 0.26: 0.5, 0.5: 0.5, 0.75: 1.0, 1.25: 1.0,
             1.3: 1.5, 1.75: 2.0, 2.5: 2.0, 2.6: 3.0, 3.5: 4.0, 4.9: 4.0, 5.0: 4.0, 5.1: 6.0,
             6.0: 6.0, 7.9: 6.0, 100.0: 6.0}
    for x, want in cases.items():
        assert fp4_round(np.array([x]))[0] == want, x
        assert fp4_round(np.array([-x]))[0] == -want, -x


def test_fp4_round_is_nearest_on_the_grid():
    rng = np.random.default_rng(0)
    y = rng.uniform(-6, 6, 5000)
    r = fp4_round(y)
    full = np.concatenate([-FP4_GRID[::-1], FP4_GRID])
    best = np.abs(y[:, None] - full[None, :]).min(axis=1)
    assert np.all(np.abs(np.abs(y - r) - best) < 1e-12)


def test_mxfp4_exponent_rule_and_grid_values():
    rng = np.random.default_rng(1)
    for e in (-6, 0, 3):
        vals = rng.choice(np.concatenate([-FP4_GRID, FP4_GRID]), 32)
        vals[5] = 6.0  # amax 6 * 2^e: shared exponent floor(log2(6 * 2^e)) - 2 = e
        x = vals * 2.0 ** e
        v, ex = mxfp4_quantize(x[None])
        assert ex[0, 0] == e
        assert np.array_equal(mxfp4_dequantize(v, ex)[0], x)


def test_mxfp4_error_bound_and_saturation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128)).astype(np.float32).astype(np.float64)
    v, ex = mxfp4_quantize(x)
    dq = mxfp4_dequantize(v, ex)
    scale = np.repeat(np.exp2(ex.astype(np.float64)), 32, axis=-1)
    y = x / scale
    # grid spacing around |y| (0.5 below 2, 1 below 4, 2 above), halved;
    # above 6 the saturation error |y| - 6 (< 2, since amax / 2^E < 8)
    a = np.abs(y)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a > 6, a - 6, half) * scale
    assert np.all(np.abs(dq - x) <= bound + 1e-15)
    assert np.all(np.abs(v) <= 6)
    z, ez = mxfp4_quantize(np.zeros((1, 32)))
    assert np.all(z == 0) and ez[0, 0] == -127


def test_scores_brute_force():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype="bf16", causal=True, seed=71,
                     k_offset_std=3.0)
    sc = lowbit_scores(t["q"], t["k"], 2, 1, True)
    qd, kd = lowbit_inputs(t["q"], t["k"])
    for h in range(2):
        for i in range(2):
            for j in range(4):
                best = -math.inf
                for r in range(128 * i, 128 * i + 128):
                    for kk in range(64 * j, 64 * j + 64):
                        if kk <= r:
                            best = max(best, math.fsum(qd[0, h, r] * kd[0, 0, kk]))
                assert sc[0, h, i, j] == pytest.approx(best, rel=1e-12, abs=1e-12), (h, i, j)


def test_grid_inputs_give_exact_scores():
    # Q and smoothed K already on the MX FP4 grid (every 32-channel group holds
    # a +-6 * 2^e element): the estimates are the exact q . (k - k_mean)
    rng = np.random.default_rng(3)
    N, d = 256, 64
    full = np.concatenate([-FP4_GRID, FP4_GRID])
    q = rng.choice(full, (1, 2, N, d)) * 0.25
    q[..., ::32] = 6 * 0.25
    half = rng.choice(full, (1, 1, N // 2, d)) * 0.5
    half[..., ::32] = 6 * 0.5
    k0 = np.concatenate([half, -half], axis=2)          # channel mean 0
    tq = torch.from_numpy(q).to(torch.bfloat16)
    tk = torch.from_numpy(k0).to(torch.bfloat16)
    assert np.array_equal(tq.double().numpy(), q) and np.array_equal(tk.double().numpy(), k0)
    sc = lowbit_scores(tq, tk, 2, 1, False)
    exact = np.einsum("hnd,md->hnm", q[0], k0[0, 0])
    want = exact.reshape(2, 2, 128, 4, 64).max(axis=(2, 4))
    assert np.array_equal(sc[0], want)


def test_planted_element_wins_its_block_and_keep_extremes():
    p, t = make_case(B=1, Hq=1, Hkv=1, N=1024, d=64, dtype="bf16", causal=True, seed=72,
                     k_offset_std=1.0)
    q, k = t["q"].clone(), t["k"].clone()
    # one query row of block 7 and one key of block 5 aligned and large: block
    # (7, 5) holds the largest estimate of row block 7
    q[0, 0, 7 * 128 + 3] = 8.0
    k[0, 0, 5 * 64 + 9] = 8.0 + k[0, 0].float().mean(0).to(torch.bfloat16)
    idx, cnt, ties, sc = lowbit_block_mask(q, k, 1, 1, True, 1, 16)
    kept = list(idx[0, 0, 7, :cnt[0, 0, 7]])
    assert 5 in kept
    assert np.argmax(np.where(np.isfinite(sc[0, 0, 7]), sc[0, 0, 7], -np.inf)[:14]) == 5
    idx, cnt, _, _ = lowbit_block_mask(q, k, 1, 1, True, 1, 1)
    for i in range(8):
        assert list(idx[0, 0, i, :cnt[0, 0, i]]) == list(range(2 * i + 2))
    idx, cnt, _, _ = lowbit_block_mask(q, k, 1, 1, True, 0, 1)
    for i in range(8):
        assert list(idx[0, 0, i, :cnt[0, 0, i]]) == sorted({0, 2 * i, 2 * i + 1})
