"""Pins of the adaptive per-head precision oracle: the sampled error proxy
``head_error`` and the all-or-nothing kept lists ``adaptive_lists``.

What fixes the proxy independently of its vectorized formula:

* a brute force over the sampled pairs with scalar loops (exact integer code
  sums, math.fsum for the 16-bit logit);
* inputs whose smoothing and quantization are exact give (almost) zero error;
* scaling Q by a power of two scales the error by the same factor, exactly;
* on Gaussian inputs the error matches the uniform-rounding noise model
  E[(s8 - s16)^2] = c^2 sum_d (q_d^2 sk^2 + ks_d^2 sq^2) / 12 within a few %;
* the lists promote every visible block of a flagged head and nothing else,
  and the promoted forward with them is the dense INT8 emulation when no head
  is flagged.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import (adaptive_lists, emulate_attention, emulate_promoted_attention,
                              head_error, head_error_sample, promote_plan, softmax_scale_log2)
from synthetic import make_case


def _err(t, Hq, Hkv):
    sq = oracle.smooth_quant(t["q"], t["k"])
    return sq, head_error(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["q"], t["k"],
                          sq["k_mean"], Hq, Hkv)


def test_sample_shape_and_spread():
    rows, keys = head_error_sample(8192)
    assert len(rows) == 64 and len(keys) == 128
    assert len(set(rows // 128)) == 64 and len(set(keys // 64)) == 128
    rows, keys = head_error_sample(65536)
    assert len(rows) == 64 and len(keys) == 256
    assert np.all(np.diff(rows // 128) == 8) and np.all(np.diff(keys // 64) == 4)
    rows, keys = head_error_sample(256)
    assert list(rows // 128) == [0, 1] and list(keys // 64) == [0, 1, 2, 3]


def test_head_error_brute_force():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=384, d=64, dtype="bf16", causal=True, seed=51,
                     k_offset_std=3.0, outliers=2)
    sq, err = _err(t, 2, 1)
    rows, keys = head_error_sample(p.N)
    c = float(softmax_scale_log2(p.d))
    qf = t["q"].double().numpy()
    kf = t["k"].double().numpy()
    for h in range(2):
        tot = 0.0
        for r in rows:
            qm = math.fsum(float(qf[0, h, r, x]) * float(sq["k_mean"][0, 0, x]) for x in range(p.d))
            for kk in keys:
                S = sum(int(sq["q_i8"][0, h, r, x]) * int(sq["k_i8"][0, 0, kk, x])
                        for x in range(p.d))
                aq = np.float32(np.float32(sq["q_scale"][0, h, r // 128]) * np.float32(c))
                al = np.float32(aq * np.float32(sq["k_scale"][0, 0, kk // 64]))
                s8 = float(np.float32(np.float32(S) * al))
                qk = math.fsum(float(qf[0, h, r, x]) * float(kf[0, 0, kk, x]) for x in range(p.d))
                s16 = c * (qk - qm)
                tot += (s8 - s16) ** 2
        want = math.sqrt(tot / (len(rows) * len(keys)))
        assert abs(err[0, h] - want) <= 1e-9 * want


def test_exactly_quantizable_inputs_have_no_error():
    from test_oracle_promote import _exact_quant_case
    t, _ = _exact_quant_case("bf16")
    sq, err = _err(t, 2, 1)
    # only the fp32 rounding of the INT8 logit remains
    assert np.all(err < 1e-6)


def test_error_scales_with_q():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=128, dtype="bf16", causal=False, seed=52,
                     k_offset_std=3.0, outliers=4)
    _, e1 = _err(t, 2, 1)
    t2 = dict(t, q=t["q"] * 4)  # exact in bf16
    _, e4 = _err(t2, 2, 1)
    assert np.allclose(e4, 4 * e1, rtol=1e-12, atol=0)


@pytest.mark.parametrize("d", [64, 128])
def test_error_matches_the_rounding_noise_model(d):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=4096, d=d, dtype="bf16", causal=False, seed=53,
                     k_offset_std=2.0)
    sq, err = _err(t, 2, 1)
    rows, keys = head_error_sample(p.N)
    c = float(softmax_scale_log2(d))
    ks = t["k"].double().numpy()[0, 0] - sq["k_mean"][0, 0].astype(np.float64)
    for h in range(2):
        qr = t["q"].double().numpy()[0, h, rows]
        sqs = sq["q_scale"][0, h, rows // 128].astype(np.float64)
        sks = sq["k_scale"][0, 0, keys // 64].astype(np.float64)
        var = ((qr ** 2).sum(1)[:, None] * sks[None, :] ** 2 +
               (ks[keys] ** 2).sum(1)[None, :] * sqs[:, None] ** 2) / 12.0
        pred = c * math.sqrt(var.mean())
        assert abs(err[0, h] / pred - 1.0) < 0.05, (err[0, h], pred)


@pytest.mark.parametrize("causal", [False, True])
def test_adaptive_lists(causal):
    N = 640
    flags = np.array([[True, False, True]])
    idx, cnt = adaptive_lists(flags, N, causal)
    for h in range(3):
        for i in range(N // 128):
            low, prom = promote_plan(idx[0, h, i], int(cnt[0, h, i]), i, N, causal)
            if flags[0, h]:
                assert low == [] and len(prom) == int(cnt[0, h, i]) > 0
            else:
                assert prom == [] and cnt[0, h, i] == 0


def test_adaptive_forward_with_no_flag_is_dense_int8():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=54)
    sq = oracle.smooth_quant(t["q"], t["k"])
    idx, cnt = adaptive_lists(np.zeros((1, 2), dtype=bool), p.N, True)
    a = emulate_promoted_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["q"],
                                   t["k"], sq["k_mean"], t["v"], True, 2, 1, idx, cnt, tau=8.0)
    b = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 2,
                          1, tau=8.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
