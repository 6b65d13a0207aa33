"""Pins of the promoted-path emulation (the kept blocks at 16-bit Q K^T, the
rest through the INT8 path, one online softmax).

What fixes the result independently of the emulation's own formulas:

* the tile plan is brute-forced: the low and promoted lists partition the
  visible blocks, whatever the kept list holds (duplicates, out-of-range or
  invisible entries);
* with nothing promoted the path is the dense INT8 emulation, bit for bit;
* with every block promoted and no 16-bit rounding of P, the result is exact
  softmax attention (fp64 library routine), and lse is exact attention's lse
  shifted by q . k_mean / sqrt(d) (the smoothing's per-row constant);
* on inputs whose smoothed K and Q quantize exactly, the INT8 and 16-bit
  logits coincide, so any mix of the two paths is exact attention; handing the
  16-bit path a wrong K mean (a planted mistake) breaks that;
* closed forms: V = 1 gives 1 within V's unit roundoff; causal row 0 is V_0;
* the summary's claim, checked on a seeded case: promoting the kept blocks is
  closer to exact attention than skipping the rest, and no worse than INT8
  everywhere.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import (emulate_attention, emulate_promoted_attention, exact_attention,
                              promote_plan, softmax_scale_log2)
from synthetic import make_case


def _sq_mask(p, t, keep=(1, 10)):
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, p.causal, *keep)
    return sq, idx, cnt


def _promoted(p, t, sq, idx, cnt, **kw):
    return emulate_promoted_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                      t["q"], t["k"], sq["k_mean"], t["v"], p.causal, p.Hq, p.Hkv,
                                      idx, cnt, **kw)


@pytest.mark.parametrize("causal", [False, True])
def test_promote_plan_partitions_visible_blocks(causal):
    rng = np.random.default_rng(5)
    N = 1024
    nkb = N // 64
    for trial in range(200):
        i = int(rng.integers(0, N // 128))
        L = int(rng.integers(0, 24))
        row = rng.integers(-3, nkb + 3, L)
        cnt = int(rng.integers(0, L + 1))
        low, prom = promote_plan(row, cnt, i, N, causal)
        visible = [j for j in range(nkb) if not causal or 64 * j <= 128 * i + 127]
        kept = set(int(x) for x in row[:cnt])
        assert prom == sorted(set(visible) & kept)
        assert low == [j for j in visible if j not in kept]
        assert sorted(low + prom) == visible


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_promote_nothing_is_the_dense_int8_emulation(tau):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=3)
    sq = oracle.smooth_quant(t["q"], t["k"])
    nqb = p.N // 128
    idx = np.full((1, 2, nqb, 4), -1, dtype=np.int32)
    cnt = np.zeros((1, 2, nqb), dtype=np.int32)
    a = _promoted(p, t, sq, idx, cnt, tau=tau)
    b = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True,
                          2, 1, tau=tau)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_promote_everything_is_exact_attention(dtype, d):
    # K with large per-channel offsets: q . k_mean is far from zero, so a
    # missing or sign-flipped correction would show in lse
    p, t = make_case(B=1, Hq=2, Hkv=1, N=384, d=d, dtype=dtype, causal=True, seed=8,
                     k_offset_std=3.0, outliers=4)
    sq = oracle.smooth_quant(t["q"], t["k"])
    nqb, nkb = p.N // 128, p.N // 64
    idx = np.tile(np.arange(nkb, dtype=np.int32), (1, 2, nqb, 1))
    cnt = np.full((1, 2, nqb), nkb, dtype=np.int32)
    _, Opre, lse = _promoted(p, t, sq, idx, cnt, p_dtype="f32", tau=0.0)
    Oe, lse_e = exact_attention(t["q"], t["k"], t["v"], True)
    assert np.abs(Opre - Oe).max() <= 2e-5 * np.abs(Oe).max()
    q64 = t["q"].double().numpy()
    qm = np.einsum("bhnd,bd->bhn", q64, sq["k_mean"][:, 0].astype(np.float64))
    assert np.abs(qm / math.sqrt(d)).max() > 1.0     # the correction matters here
    assert np.abs(lse + qm / math.sqrt(d) - lse_e).max() < 2e-4


def _exact_quant_case(dtype, d=64, N=512, seed=0):
    """Q, K whose smoothing and quantization are exact (module docstring)."""
    rng = np.random.default_rng(seed)
    # Q = codes * 2^-6, every 128-row block reaching 127 * 2^-6 (scale 2^-6)
    qc = rng.integers(-8, 9, (1, 2, N, d)).astype(np.float64)
    qc[:, :, ::128, 0] = 127
    qc[:, :, ::128, 1:] = 0
    # K = K0 + m: K0 = codes * 2^-3 summing to zero per channel, every 64-token
    # block reaching 127 * 2^-3 (scale 2^-3); m = integers * 2^-3 (exact mean)
    half = rng.integers(-100, 101, (1, 1, N // 2, d)).astype(np.float64)
    half[:, :, 0::64, 1] = 127
    k0 = np.concatenate([half, -half], axis=2)
    m = rng.integers(-24, 25, (1, 1, 1, d)).astype(np.float64)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q = torch.from_numpy(qc * 2.0 ** -6).to(dt)
    k = torch.from_numpy((k0 + m) * 2.0 ** -3).to(dt)
    assert np.array_equal(q.double().numpy(), qc * 2.0 ** -6)
    assert np.array_equal(k.double().numpy(), (k0 + m) * 2.0 ** -3)
    v = torch.from_numpy(rng.standard_normal((1, 1, N, d))).to(dt)
    return {"q": q, "k": k, "v": v}, m[0, 0, 0] * 2.0 ** -3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_mixed_paths_on_exactly_quantized_inputs_are_exact(dtype, causal):
    t, mean = _exact_quant_case(dtype)
    N, d = t["q"].shape[2], t["q"].shape[3]
    sq = oracle.smooth_quant(t["q"], t["k"])
    assert np.array_equal(sq["k_mean"][0, 0].astype(np.float64), mean)
    assert np.all(sq["q_scale"] == 2.0 ** -6) and np.all(sq["k_scale"] == 2.0 ** -3)
    nqb, nkb = N // 128, N // 64
    rng = np.random.default_rng(1)
    idx = np.full((1, 2, nqb, 5), -1, dtype=np.int32)
    cnt = np.zeros((1, 2, nqb), dtype=np.int32)
    for h in range(2):
        for i in range(nqb):
            pick = sorted(rng.choice(nkb, 4, replace=False))
            idx[0, h, i, :4] = pick
            cnt[0, h, i] = 4
    args = (sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["q"], t["k"])
    tail = (t["v"], causal, 2, 1, idx, cnt)
    _, Opre, lse = emulate_promoted_attention(*args, sq["k_mean"], *tail, p_dtype="f32")
    Oe, lse_e = exact_attention(t["q"], t["k"], t["v"], causal)
    vmax = float(t["v"].abs().max())
    assert np.abs(Opre - Oe).max() <= 1e-5 * vmax
    # a planted mistake: the 16-bit path told the K mean is zero
    _, Obad, _ = emulate_promoted_attention(*args, np.zeros_like(sq["k_mean"]), *tail,
                                            p_dtype="f32")
    assert np.abs(Obad - Oe).max() > 1e-2 * vmax


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_promoted_v_ones_gives_ones(dtype):
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype=dtype, causal=True, seed=4)
    t["v"] = torch.ones_like(t["v"])
    sq, idx, cnt = _sq_mask(p, t, keep=(1, 4))
    O, Opre, _ = _promoted(p, t, sq, idx, cnt, tau=8.0)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.abs(Opre - 1.0).max() <= u * (1 + 1e-6)
    assert np.abs(O - 1.0).max() <= u


def test_promoted_causal_row_zero_is_v0():
    p, t = make_case(B=1, Hq=2, Hkv=2, N=256, d=64, dtype="bf16", causal=True, seed=6)
    sq, idx, cnt = _sq_mask(p, t)
    O, _, _ = _promoted(p, t, sq, idx, cnt)
    assert np.array_equal(O[0, :, 0], t["v"][0, :, 0].float().numpy())


def test_promote_beats_skip_and_matches_or_beats_int8():
    # Llama-shaped law (large per-channel K offsets, outlier channels)
    p, t = make_case(B=1, Hq=4, Hkv=1, N=1024, d=128, dtype="bf16", causal=True, seed=21,
                     k_offset_std=3.0, outliers=4)
    sq, idx, cnt = _sq_mask(p, t, keep=(1, 10))
    Oe, _ = exact_attention(t["q"], t["k"], t["v"], True)
    O_prom, _, _ = _promoted(p, t, sq, idx, cnt, tau=8.0)
    args = (sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 4, 1)
    O_dense, _, _ = emulate_attention(*args, tau=8.0)
    O_skip, _, _ = emulate_attention(*args, kv_idx=idx, kv_cnt=cnt, tau=8.0)

    def rms(x):
        return float(np.sqrt(np.mean((x - Oe) ** 2)))

    assert rms(O_prom) < 0.5 * rms(O_skip)
    assert rms(O_prom) <= rms(O_dense) * 1.001


def test_promoted_logit_scale_is_the_int8_scale():
    # both paths fold the same fl32(log2(e)/sqrt(d)): on exactly quantized
    # inputs a promoted half and the INT8 tile give bit-identical logits, so
    # with one kept block per query block the result is order-independent up
    # to rounding only -- checked against the dense INT8 emulation
    t, _ = _exact_quant_case("bf16", N=256)
    sq = oracle.smooth_quant(t["q"], t["k"])
    idx = np.zeros((1, 2, 2, 1), dtype=np.int32)
    cnt = np.ones((1, 2, 2), dtype=np.int32)
    _, a, la = emulate_promoted_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                          t["q"], t["k"], sq["k_mean"], t["v"], False, 2, 1,
                                          idx, cnt, p_dtype="f32")
    _, b, lb = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
                                 False, 2, 1, p_dtype="f32")
    assert np.abs(a - b).max() <= 1e-6 * np.abs(b).max()
    assert np.abs(la - lb).max() < 1e-6
    assert softmax_scale_log2(64) == np.float32(math.log2(math.e) / 8)
