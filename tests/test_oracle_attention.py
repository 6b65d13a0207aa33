"""Pins of the oracle's exact attention and of the quantized-path emulation.

Exact attention is pinned to a library routine (torch's scaled-dot-product
attention in fp64) and to a pure-Python brute force. The emulation is pinned by
closed forms (V = 1, causal row 0, constant keys), the exact-quantization
special case, shift invariance of the smoothing, the online merge against a
single-tile softmax, and the accuracy claim against exact attention.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import exact_attention, emulate_attention, softmax_scale_log2
from synthetic import make_case, make_config


def _cos(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def _emulate(p, t, **kw):
    sq = oracle.smooth_quant(t["q"], t["k"])
    return emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
                             p.causal, p.Hq, p.Hkv, **kw), sq


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (4, 1)])
def test_exact_matches_torch_sdpa_fp64(causal, Hq, Hkv):
    p, t = make_case(B=2, Hq=Hq, Hkv=Hkv, N=256, d=64, dtype="bf16", seed=3)
    O, lse = exact_attention(t["q"], t["k"], t["v"], causal)
    q, k, v = (t[x].double() for x in "qkv")
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    assert np.abs(O - ref.numpy()).max() < 1e-12
    s = (q @ k.transpose(-1, -2)) / math.sqrt(64)
    if causal:
        s = s.masked_fill(torch.ones(256, 256, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() < 1e-12


def test_exact_matches_brute_force_loops():
    rng = np.random.default_rng(0)
    N, d = 128, 8
    q = torch.from_numpy(rng.standard_normal((1, 1, N, d))).to(torch.float16)
    k = torch.from_numpy(rng.standard_normal((1, 1, N, d))).to(torch.float16)
    v = torch.from_numpy(rng.standard_normal((1, 1, N, d))).to(torch.float16)
    O, _ = exact_attention(q, k, v, True)
    qq, kk, vv = (x[0, 0].double().tolist() for x in (q, k, v))
    for i in (0, 1, 17, 127):
        w = [math.exp(sum(a * b for a, b in zip(qq[i], kk[j])) / math.sqrt(d)) for j in range(i + 1)]
        z = sum(w)
        for c in range(d):
            ref = sum(w[j] * vv[j][c] for j in range(i + 1)) / z
            assert abs(O[0, 0, i, c] - ref) < 1e-12


def test_exact_block_mask_restricts_keys():
    p, t = make_case(B=1, Hq=1, Hkv=1, N=256, d=64, dtype="bf16", seed=8)
    idx = np.full((1, 1, 2, 4), -1, dtype=np.int32)
    cnt = np.array([[[2, 3]]], dtype=np.int32)
    idx[0, 0, 0, :2] = [0, 1]
    idx[0, 0, 1, :3] = [0, 2, 3]
    O, _ = exact_attention(t["q"], t["k"], t["v"], True, idx, cnt)
    q, k, v = (t[x][0, 0].double().numpy() for x in "qkv")
    r = 200
    keys = [j for j in range(r + 1) if j < 64 or j >= 128]
    s = q[r] @ k[keys].T / 8.0
    w = np.exp(s - s.max())
    assert np.abs(O[0, 0, r] - w @ v[keys] / w.sum()).max() < 1e-12


def test_exact_smoothing_invariance():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype="f16", seed=1)
    O0, _ = exact_attention(t["q"], t["k"], t["v"], True)
    shift = torch.from_numpy(np.random.default_rng(2).standard_normal((1, 1, 1, 64)) * 4)
    k1 = (t["k"].double() + shift)
    O1, _ = exact_attention(t["q"], k1, t["v"], True)
    assert np.abs(O0 - O1).max() < 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_emulation_v_ones_gives_ones(dtype, causal):
    # O = sum(P_hat) / sum(P) with |P_hat - P| <= u P (u: unit roundoff of the
    # 16-bit type), so |O - 1| <= u; a dropped or doubled correction factor in
    # acc or l would break it by far more
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype=dtype, causal=causal, seed=4)
    t["v"] = torch.ones_like(t["v"])
    (O, Opre, _), _ = _emulate(p, t)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.all(np.abs(Opre.astype(np.float64) - 1.0) <= u * (1 + 1e-6))
    assert np.all(np.abs(O.astype(np.float64) - 1.0) <= u)


def test_emulation_causal_row_zero_is_v0():
    p, t = make_case(B=1, Hq=4, Hkv=2, N=256, d=128, dtype="bf16", causal=True, seed=6)
    (O, _, _), _ = _emulate(p, t)
    v = t["v"].float().numpy()
    for hq in range(4):
        assert np.array_equal(O[0, hq, 0], v[0, hq // 2, 0])


def test_emulation_constant_keys_average_visible_values():
    p, t = make_case(B=1, Hq=1, Hkv=1, N=256, d=64, dtype="f16", causal=True, seed=7)
    t["k"] = t["k"][:, :, :1].expand(-1, -1, 256, -1).contiguous()
    (O, _, _), sq = _emulate(p, t)
    assert not sq["k_i8"].any()
    v = t["v"][0, 0].double().numpy()
    mean = np.cumsum(v, axis=0) / np.arange(1, 257)[:, None]
    want = oracle.f16_rne(mean.astype(np.float32))
    assert np.abs(O[0, 0] - want).max() <= np.abs(want).max() * 2 ** -10


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_emulation_exact_quantization_case_matches_exact_attention(dtype):
    # integer Q, K with exact codes and unit scales: the only difference left
    # between the emulation and exact attention is the rounding of P (and the
    # exp2/fp32 details), so the error is bounded by P's 16-bit rounding.
    rng = np.random.default_rng(0)
    N, d = 256, 64
    # small integer Q keeps most logits moderate; the first row of each query
    # block is 127 * e_0 so that every Q block's amax, hence its scale, is 1
    q = rng.integers(-2, 3, (1, 1, N, d)).astype(np.float64)
    q[0, 0, ::128, 0] = 127
    q[0, 0, ::128, 1:] = 0
    # K channels sum to zero (mean 0) and every 64-token block reaches 127
    half = rng.integers(-120, 121, (1, 1, N // 2, d)).astype(np.float64)
    half[0, 0, 0::64, 1] = 127
    k = np.concatenate([half, -half], axis=2)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = {"q": torch.from_numpy(q).to(dt), "k": torch.from_numpy(k).to(dt),
         "v": torch.from_numpy(rng.standard_normal((1, 1, N, d))).to(dt)}
    sq = oracle.smooth_quant(t["q"], t["k"])
    assert np.all(sq["k_scale"] == 1)
    O, Opre, _ = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                   t["v"], False, 1, 1)
    assert np.all(sq["q_scale"] == 1)
    Oe, _ = exact_attention(t["q"], t["k"], t["v"], False)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    # each weight is off by at most u relative, so O is off by at most 2u*max|V|
    vmax = float(t["v"].abs().max())
    assert np.abs(Opre - Oe).max() <= 2 * u * vmax + 1e-5


def test_online_merge_equals_single_tile_softmax():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=12)
    sq = oracle.smooth_quant(t["q"], t["k"])
    args = (sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 2, 1)
    _, a, la = emulate_attention(*args, kv_tile=64, p_dtype="f32")
    _, b, lb = emulate_attention(*args, kv_tile=512, p_dtype="f32")
    _, c, lc = emulate_attention(*args, kv_tile=128, p_dtype="f32")
    assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max()
    assert np.abs(c - b).max() <= 1e-5 * np.abs(b).max()
    assert np.abs(la - lb).max() < 1e-5
    # a direct two-pass softmax over the dequantized scores
    q = sq["q_i8"][0, 1].astype(np.float64)
    k = sq["k_i8"][0, 0].astype(np.float64)
    cst = softmax_scale_log2(64)
    S = q @ k.T
    alpha = (np.repeat(sq["q_scale"][0, 1], 128)[:, None] * cst).astype(np.float32) \
        * np.repeat(sq["k_scale"][0, 0], 64)[None, :]
    s = (S.astype(np.float32) * alpha.astype(np.float32)).astype(np.float64)
    s[np.triu_indices(512, 1)] = -np.inf
    w = np.exp2(s - s.max(axis=1, keepdims=True))
    ref = (w @ t["v"][0, 0].double().numpy()) / w.sum(axis=1, keepdims=True)
    assert np.abs(a[0, 1] - ref).max() <= 1e-5 * np.abs(ref).max()


def test_emulation_smoothing_invariance_bit_identical():
    rng = np.random.default_rng(9)
    kq = np.round(rng.standard_normal((1, 1, 256, 64)) * 8) / 8
    c = np.round(rng.standard_normal((1, 1, 1, 64)) * 4) / 4
    q = torch.from_numpy(rng.standard_normal((1, 2, 256, 64))).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, 1, 256, 64))).to(torch.bfloat16)
    outs = []
    for kk in (kq, kq + c):
        sq = oracle.smooth_quant(q, torch.from_numpy(kk).to(torch.bfloat16))
        outs.append(emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
                                      v, True, 2, 1)[0])
    assert np.array_equal(outs[0], outs[1])


def test_smoothing_is_what_makes_the_quantized_path_accurate():
    # the Llama-shaped law: large per-channel K offsets with x20 outlier channels
    p, t = make_config(2, N=1024)
    p = dataclasses.replace(p, Hq=8, Hkv=2)
    sub = {x: t[x][:, :8] if x == "q" else t[x][:, :2] for x in "qkv"}
    (O, _, _), sq = _emulate(p, sub)
    Oe, _ = exact_attention(sub["q"], sub["k"], sub["v"], True)
    assert _cos(O, Oe) >= 0.999
    # the same path without the mean subtraction (per-block INT8 of raw K)
    k32 = sub["k"].float().numpy()
    k_i8 = np.empty(k32.shape, dtype=np.int8)
    k_sc = np.empty((1, 2, 16), dtype=np.float32)
    for h in range(2):
        for j in range(16):
            k_i8[0, h, 64 * j:64 * j + 64], k_sc[0, h, j] = oracle.quantize_block(k32[0, h, 64 * j:64 * j + 64])
    O_raw, _, _ = emulate_attention(sq["q_i8"], sq["q_scale"], k_i8, k_sc, sub["v"], True, 8, 2)
    assert _cos(O_raw, Oe) < _cos(O, Oe)


def test_emulation_sparse_keep_all_equals_dense():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=13)
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], 2, 1, True, 1, 1)
    args = (sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 2, 1)
    dense = emulate_attention(*args)[0]
    sparse = emulate_attention(*args, kv_idx=idx, kv_cnt=cnt)[0]
    assert np.array_equal(dense, sparse)


def test_emulation_lse_matches_exact_lse_of_smoothed_logits():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=128, dtype="bf16", causal=True, seed=14,
                     k_offset_std=3.0)
    (O, _, lse), sq = _emulate(p, t)
    ks = t["k"].double() - torch.from_numpy(sq["k_mean"].astype(np.float64))[:, :, None, :]
    _, lse_e = exact_attention(t["q"], ks, t["v"], True)
    # quantization error of the logits, not rounding, sets this bound
    assert np.abs(lse - lse_e).max() < 0.05


@pytest.mark.parametrize("tau", [1.0, 8.0, 20.0])
def test_online_reference_threshold_changes_nothing_exactly(tau):
    # with unrounded P the exponent reference cancels between acc and l: any
    # threshold gives the single-tile (two-pass) result up to fp32 rounding
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=128, dtype="bf16", causal=True, seed=15,
                     k_offset_std=3.0, outliers=4)
    sq = oracle.smooth_quant(t["q"], t["k"])
    args = (sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True, 2, 1)
    _, a, la = emulate_attention(*args, p_dtype="f32", tau=tau)
    _, b, lb = emulate_attention(*args, kv_tile=512, p_dtype="f32")
    assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max()
    assert np.abs(la - lb).max() < 1e-5
    # with 16-bit P the difference is the rounding of P at other scales only
    a16 = emulate_attention(*args, tau=tau)[1]
    b16 = emulate_attention(*args)[1]
    assert np.abs(a16 - b16).max() <= 2 * 2.0 ** -8 * np.abs(b16).max()


def test_online_reference_threshold_keeps_closed_forms():
    p, t = make_case(B=1, Hq=2, Hkv=1, N=256, d=64, dtype="bf16", causal=True, seed=16)
    sq = oracle.smooth_quant(t["q"], t["k"])
    ones = torch.ones_like(t["v"])
    O1 = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], ones, True,
                           2, 1, tau=8.0)[1]
    assert np.all(np.abs(O1.astype(np.float64) - 1.0) <= 2.0 ** -8 * (1 + 1e-6))
    O = emulate_attention(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"], True,
                          2, 1, tau=8.0)[0]
    assert np.array_equal(O[0, 0, 0], t["v"][0, 0, 0].float().numpy())
