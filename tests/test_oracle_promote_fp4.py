"""Pins of the MX FP4 low path of promote instead of skip
(oracle.promote_fp4.emulate_promoted_fp4_attention).

* On inputs whose Q and smoothed K lie on the MX FP4 grid (each 32-channel
  group holds E2M1 values times 2^E with one element at 6 * 2^E, so the MX
  shared exponent is E and the codes are the values), with a per-channel K
  mean that is exact in bf16 and cancels exactly, the 4-bit products are the
  exact ones: without P's 16-bit rounding the emulation is exact attention
  (fp32 rounding only), whatever is promoted.
* A planted mistake, the low path fed unsmoothed keys, breaks that by far.
* Everything promoted runs no low tile: bit for bit the INT8-low emulation
  with everything promoted.
* V = 1 gives O = sum(P_hat) / sum(P); causal row 0 gives V_0.
* On the Llama-shaped law the 4-bit low path is far closer to exact attention
  than skipping the low blocks.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import promote_fp4
from oracle.promote_fp4 import emulate_promoted_fp4_attention
from synthetic import make_case

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _on_grid(gen, rows, d):
    """[rows, d] with every 32-channel group on the MX FP4 grid at its own
    exponent E in [-3, 0] (one element of each group is +-6 * 2^E)."""
    v = GRID[gen.integers(0, 8, (rows, d))] * np.where(gen.random((rows, d)) < 0.5, -1.0, 1.0)
    g = v.reshape(rows, d // 32, 32)
    g[:, :, 0] = 6.0 * np.where(gen.random((rows, d // 32)) < 0.5, -1.0, 1.0)
    e = gen.integers(-3, 1, (rows, d // 32, 1))
    return (g * np.exp2(e)).reshape(rows, d)


def _grid_case(seed=3, N=512, d=128, causal=True, mean=True):
    gen = np.random.default_rng(seed)
    Hq, Hkv = 2, 1
    q = np.stack([_on_grid(gen, N, d) for _ in range(Hq)])[None]
    half = _on_grid(gen, N // 2, d)
    k0 = np.concatenate([half, -half])                  # channel sums exactly 0
    c = (gen.integers(-64, 65, d) / 16.0) if mean else np.zeros(d)   # multiples of 2^-4
    k = (k0 + c[None, :])[None, None]
    v = gen.standard_normal((1, Hkv, N, d))
    t = {x: torch.from_numpy(a).to(torch.bfloat16) for x, a in (("q", q), ("k", k), ("v", v))}
    assert torch.equal(t["q"].double(), torch.from_numpy(q))
    assert torch.equal(t["k"].double(), torch.from_numpy(k))
    return t, Hq, Hkv, N, causal


def _lists(Hq, N, promoted):
    """kv_idx/kv_cnt promoting the given block set in every query block."""
    nqb = N // 128
    idx = np.full((1, Hq, nqb, max(1, len(promoted))), -1, dtype=np.int32)
    cnt = np.zeros((1, Hq, nqb), dtype=np.int32)
    for h in range(Hq):
        for i in range(nqb):
            idx[0, h, i, :len(promoted)] = promoted
            cnt[0, h, i] = len(promoted)
    return idx, cnt


@pytest.mark.parametrize("promoted", [[], [0, 3, 5], list(range(8))])
def test_on_grid_is_exact_attention(promoted):
    t, Hq, Hkv, N, causal = _grid_case()
    sq = oracle.smooth_quant(t["q"], t["k"])
    assert np.all(sq["k_mean"][0, 0] == np.asarray(
        t["k"][0, 0].double().mean(0), dtype=np.float32))
    idx, cnt = _lists(Hq, N, promoted)
    _, o_pre, lse = emulate_promoted_fp4_attention(t["q"], t["k"], sq["k_mean"], t["v"], causal,
                                                   Hq, Hkv, idx, cnt, p_dtype="f32")
    o_ex, lse_ex = oracle.exact_attention(t["q"], t["k"], t["v"], causal)
    # the logits are exact up to one fp32 rounding each
    assert np.abs(o_pre - o_ex).max() <= 2e-5 * np.abs(o_ex).max()
    # lse of the smoothed logits: exact lse shifted by q . k_mean / sqrt(d)
    qm = t["q"][0].double().numpy() @ sq["k_mean"][0, 0].astype(np.float64)
    assert np.abs(lse - (lse_ex - qm / np.sqrt(128))).max() < 1e-4


def test_planted_unsmoothed_low_path_breaks_the_closed_form(monkeypatch):
    t, Hq, Hkv, N, causal = _grid_case(seed=4)
    sq = oracle.smooth_quant(t["q"], t["k"])
    idx, cnt = _lists(Hq, N, [1, 2])
    real = promote_fp4.lowbit_inputs
    # the mistake: the low path's K codes from the raw, unsmoothed K
    monkeypatch.setattr(promote_fp4, "lowbit_inputs",
                        lambda q, k, km: real(q, k, np.zeros_like(np.asarray(km))))
    _, o_bad, _ = emulate_promoted_fp4_attention(t["q"], t["k"], sq["k_mean"], t["v"], causal,
                                                 Hq, Hkv, idx, cnt, p_dtype="f32")
    o_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], causal)
    assert np.abs(o_bad - o_ex).max() > 0.05 * np.abs(o_ex).max()


def test_everything_promoted_is_the_int8_variant_bit_for_bit():
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=64, dtype="bf16", causal=True, seed=5,
                     k_offset_std=3.0)
    sq = oracle.smooth_quant(t["q"], t["k"])
    nqb, nkb = p.N // 128, p.N // 64
    idx = np.broadcast_to(np.arange(nkb, dtype=np.int32), (1, p.Hq, nqb, nkb)).copy()
    cnt = np.full((1, p.Hq, nqb), nkb, dtype=np.int32)
    a = emulate_promoted_fp4_attention(t["q"], t["k"], sq["k_mean"], t["v"], True, p.Hq, p.Hkv,
                                       idx, cnt, tau=8.0)
    b = oracle.emulate_promoted_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                          t["q"], t["k"], sq["k_mean"], t["v"], True, p.Hq, p.Hkv,
                                          idx, cnt, tau=8.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_v_ones_and_causal_row0(dtype):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=384, d=128, dtype=dtype, causal=True, seed=6,
                     k_offset_std=3.0, outliers=2)
    sq = oracle.smooth_quant(t["q"], t["k"])
    idx, cnt = _lists(2, p.N, [0, 4])
    t1 = dict(t, v=torch.ones_like(t["v"]))
    o, o_pre, _ = emulate_promoted_fp4_attention(t1["q"], t1["k"], sq["k_mean"], t1["v"], True, 2,
                                                 1, idx, cnt, tau=8.0)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.abs(o_pre.astype(np.float64) - 1.0).max() <= u
    o, _, _ = emulate_promoted_fp4_attention(t["q"], t["k"], sq["k_mean"], t["v"], True, 2, 1,
                                             idx, cnt, tau=8.0)
    v0 = t["v"][0, 0, 0].float().numpy()
    assert np.array_equal(o[0, 0, 0], v0) and np.array_equal(o[0, 1, 0], v0)


def test_fp4_low_path_beats_skip_on_the_llama_law():
    p, t = make_case(B=1, Hq=4, Hkv=1, N=1024, d=128, dtype="bf16", causal=True, seed=7,
                     k_offset_std=3.0, outliers=4)
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, True, 1, 10)
    o4, _, _ = emulate_promoted_fp4_attention(t["q"], t["k"], sq["k_mean"], t["v"], True, p.Hq,
                                              p.Hkv, idx, cnt, tau=8.0)
    o_skip, _, _ = oracle.emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                            t["v"], True, p.Hq, p.Hkv, kv_idx=idx, kv_cnt=cnt,
                                            tau=8.0)
    o_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], True)

    def rms(o):
        return float(np.sqrt(np.mean((o.astype(np.float64) - o_ex) ** 2)))

    assert rms(o4) < 0.5 * rms(o_skip)
