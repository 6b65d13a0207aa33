"""Pins of the oracle's smoothing and quantization (CPU only).

Each test fixes a property that the definitions imply independently of how the
oracle computes them: exact rationals, closed forms, ties, shift invariance.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.quant import quantize_block, k_channel_mean, smooth_quant, q_block_pool, k_block_pool
from synthetic import make_case


def _fl32_of_fraction(fr: Fraction) -> np.float32:
    """fl32(fl64(fr)): the oracle's stated two-step rounding of a rational."""
    return np.float32(float(fr))


def test_quantizer_round_trip_bound():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        codes, scale = quantize_block(x)
        assert codes.dtype == np.int8
        assert np.all(np.abs(codes.astype(int)) <= 127)
        err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * np.float64(scale))
        # half a step, plus the fp32 rounding of the scale itself
        assert np.all(err <= 0.5 * scale * (1 + 2.0 ** -20) + 127 * scale * 2.0 ** -23)
        # the element of largest magnitude maps to +-127
        a = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert abs(int(codes[a])) == 127
        assert scale == np.float32(np.float32(np.max(np.abs(x))) / np.float32(127))


def test_quantizer_ties_to_even_and_exact_codes():
    # amax = 127 makes the scale exactly 1.0, so codes are the rounded values
    x = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, 0.49999997],
                 dtype=np.float32)
    codes, scale = quantize_block(x)
    assert scale == np.float32(1.0)
    assert codes.tolist() == [127, 2, 4, -2, -4, 0, 2, 0, 126, 0]


def test_quantizer_zero_block():
    codes, scale = quantize_block(np.zeros((64, 64), dtype=np.float32))
    assert scale == np.float32(1.0)
    assert not codes.any()


def test_quantizer_rounds_the_exact_quotient():
    # x / scale whose float32 quotient rounds onto a half-integer while the exact
    # quotient lies off it: the code follows the exact quotient.
    rng = np.random.default_rng(11)
    hits = 0
    for _ in range(4000):
        amax = np.float32(rng.uniform(1, 100))
        s = np.float32(amax / np.float32(127))
        k = int(rng.integers(0, 126))
        x = np.float32((k + 0.5) * float(s))
        for cand in (x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))):
            if cand > amax:
                continue
            exact = Fraction(float(cand)) / Fraction(float(s))
            half = Fraction(2 * k + 1, 2)
            if exact != half and np.float32(cand / s) == np.float32(k + 0.5):
                codes, sc = quantize_block(np.array([amax, cand], dtype=np.float32))
                assert sc == s
                assert int(codes[1]) == (k + 1 if exact > half else k)
                hits += 1
    assert hits > 10


def test_k_mean_is_rounded_exact_mean():
    p, t = make_case(B=1, Hq=2, Hkv=2, N=512, d=64, dtype="bf16", seed=5, k_offset_std=3.0,
                     outliers=4)
    k = t["k"].to(torch.float64).numpy()
    m = k_channel_mean(t["k"])
    for h in range(2):
        for c in range(0, 64, 7):
            exact = sum((Fraction(float(a)) for a in k[0, h, :, c]), Fraction(0)) / 512
            assert m[0, h, c] == _fl32_of_fraction(exact)


def test_smoothing_removes_a_per_channel_shift_exactly():
    # K on a coarse dyadic grid, so K + c, the sums and the means are all exact:
    # shifting every token of a channel by c must leave the smoothed K, and so
    # every code and scale, bit-identical.
    rng = np.random.default_rng(9)
    kq = np.round(rng.standard_normal((1, 2, 256, 64)) * 8) / 8
    c = np.round(rng.standard_normal((1, 2, 1, 64)) * 4) / 4
    q = torch.from_numpy(rng.standard_normal((1, 2, 256, 64))).to(torch.bfloat16)
    k0 = torch.from_numpy(kq).to(torch.bfloat16)
    k1 = torch.from_numpy(kq + c).to(torch.bfloat16)
    assert torch.equal(k1.double() - k0.double(), torch.from_numpy(np.broadcast_to(c, kq.shape).copy()).double())
    a = smooth_quant(q, k0)
    b = smooth_quant(q, k1)
    assert np.array_equal(b["k_mean"], (a["k_mean"] + c[:, :, 0, :].astype(np.float32)))
    assert np.array_equal(a["k_i8"], b["k_i8"])
    assert np.array_equal(a["k_scale"], b["k_scale"])


def test_smoothed_k_has_zero_channel_mean_and_smaller_scale():
    p, t = make_case(B=1, Hq=4, Hkv=2, N=1024, d=128, dtype="bf16", seed=2,
                     k_offset_std=3.0, outliers=4)
    sq = smooth_quant(t["q"], t["k"])
    k = t["k"].to(torch.float64).numpy()
    ks = k.astype(np.float32) - sq["k_mean"][:, :, None, :]
    assert np.abs(ks.astype(np.float64).mean(axis=2)).max() < 1e-5
    # without smoothing the outlier channels set the scale; with it the noise does
    raw_scale = np.abs(k).reshape(1, 2, 16, 64, 128).max(axis=(3, 4)) / 127
    assert np.all(sq["k_scale"] < raw_scale)


def test_pools_are_rounded_block_means():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype="bf16", seed=4,
                     k_offset_std=3.0)
    q = t["q"].to(torch.float64).numpy()
    k = t["k"].to(torch.float64).numpy()
    m = k_channel_mean(t["k"])
    qp = q_block_pool(t["q"])
    kp = k_block_pool(t["k"], m)
    for i in range(2):
        for c in (0, 5, 63):
            ex = sum((Fraction(float(a)) for a in q[0, 1, 128 * i:128 * i + 128, c]), Fraction(0)) / 128
            assert qp[0, 1, i, c] == _fl32_of_fraction(ex)
    for j in range(4):
        for c in (1, 17, 62):
            ex = sum((Fraction(float(a)) for a in k[0, 0, 64 * j:64 * j + 64, c]), Fraction(0)) / 64
            want = np.float32(float(ex) - float(m[0, 0, c]))
            assert kp[0, 0, j, c] == want


def test_pool_vector_quant_is_block_rule_per_vector():
    rng = np.random.default_rng(1)
    p = rng.standard_normal((5, 3, 64)).astype(np.float32)
    codes, scales = oracle.pool_vector_quant(p)
    for a in range(5):
        for b in range(3):
            c, s = quantize_block(p[a, b])
            assert np.array_equal(c, codes[a, b]) and s == scales[a, b]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_exact_integer_inputs_quantize_to_themselves(dtype):
    # integer-valued Q and K in [-127, 127], every block reaching 127 and every K
    # channel summing to 0: codes equal the values and every scale is 1.
    rng = np.random.default_rng(0)
    q = rng.integers(-127, 128, (1, 1, 256, 64)).astype(np.float64)
    q[0, 0, ::128, 0] = 127
    half = rng.integers(-120, 121, (1, 1, 128, 64)).astype(np.float64)
    half[0, 0, 0::64, 1] = 127     # K blocks 0, 1 reach +127; blocks 2, 3 reach -127
    k = np.concatenate([half, -half], axis=2)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    sq = smooth_quant(torch.from_numpy(q).to(dt), torch.from_numpy(k).to(dt))
    assert not sq["k_mean"].any()
    assert np.array_equal(sq["q_i8"].astype(np.float64), q)
    assert np.array_equal(sq["k_i8"].astype(np.float64), k)
    assert np.all(sq["q_scale"] == 1) and np.all(sq["k_scale"] == 1)
