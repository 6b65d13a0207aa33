"""Pins of the oracle's rounding helpers against library casts and exact rationals."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.rounding import bf16_rne, f16_rne, exact_sum


def _edge_values():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(50)
    # exact bf16 ties: halfway between two bf16 values, both parities
    base = np.array([1.0, 1.0078125, 3.0, -5.5, 1e-30, 65280.0], dtype=np.float32)
    u = base.view(np.uint32)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    near = np.concatenate([(u | np.uint32(0x7FFF)).view(np.float32),
                           (u | np.uint32(0x8001)).view(np.float32)])
    special = np.array([0.0, -0.0, 3.3895314e38, 1e-40, -1e-42, 65504.0, 65520.0, 6e-8],
                       dtype=np.float32)
    return np.concatenate([x, ties, near, special])


def test_bf16_rne_matches_torch_cast():
    x = _edge_values()
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = bf16_rne(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_f16_rne_matches_torch_cast():
    x = _edge_values()
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float32).numpy()
    got = f16_rne(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_rne_ties_to_even_by_hand():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: even mantissa is 1.0
    assert bf16_rne(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert bf16_rne(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_sum_is_correctly_rounded(seed):
    rng = np.random.default_rng(seed)
    # values spanning a wide exponent range, where naive fp64 summation rounds
    v = rng.standard_normal(4096) * np.exp2(rng.integers(-60, 40, 4096))
    v = np.concatenate([v, [1e30, -1e30, 2 ** -70]])
    exact = sum((Fraction(float(a)) for a in v), Fraction(0))
    got = exact_sum(v)
    # float() of a Fraction is the correctly rounded double of the rational
    assert float(exact) == got
