"""GPU parity of the vertical / slash pattern prediction
(qattn_block_mask_patterns) against oracle.patterns.predict_patterns, through
the C ABI.

The lines and the extended lists are integer work: compared bit for bit.
Inputs are seeded random lists (duplicates, invalid entries, counts past
max_keep), the oracle's own masks (pooled and element-level 4-bit) at small
sizes and the pooled mask at the full N = 32768 size; the whole chain (each
side's own mask, then its own prediction) is compared where the two masks
agree; the block-sparse forward over the extended lists is compared with the
emulation under the same bars as the other forwards.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.patterns import predict_patterns
from synthetic import make_case, make_config
from parity_util import log, to_np, same_lists, emulate_both, check_out

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _gpu_patterns(qa, p, idx, cnt, nv, ns, mk_out=None):
    B, Hq, nqb, mk = idx.shape
    nkb = p.N // 64
    if mk_out is None:
        mk_out = min(nkb, mk + nv + ns)
    oi = torch.full((B, Hq, nqb, mk_out), 12345, dtype=torch.int32, device=DEV)
    oc = torch.full((B, Hq, nqb), 12345, dtype=torch.int32, device=DEV)
    lines = torch.full((B, Hq, max(1, nv + ns)), 777, dtype=torch.int32, device=DEV)
    qa.qattn_block_mask_patterns(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal),
                                 torch.from_numpy(np.ascontiguousarray(idx)).to(DEV),
                                 torch.from_numpy(np.ascontiguousarray(cnt)).to(DEV), mk, nv, ns,
                                 oi, oc, mk_out, lines)
    torch.cuda.synchronize()
    return to_np(lines)[..., :nv + ns].astype(np.int64), to_np(oi).astype(np.int64), \
        to_np(oc).astype(np.int64)


def _check(got, want):
    gl, gi, gc = got
    wl, wi, wc = want
    assert np.array_equal(gl, wl), "lines"
    assert np.array_equal(gc, wc), "counts"
    assert np.array_equal(gi, wi), "lists"


class _P:
    def __init__(self, B, Hq, Hkv, N, d, dtype, causal):
        self.B, self.Hq, self.Hkv, self.N, self.d, self.dtype, self.causal = \
            B, Hq, Hkv, N, d, dtype, causal


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,mk,nv,ns", [(2048, 9, 4, 4), (8192, 20, 8, 6), (640, 5, 64, 64),
                                        (4096, 12, 0, 0), (131072, 30, 16, 16)])
def test_random_lists_bit_exact(gpu_lib, causal, N, mk, nv, ns):
    rng = np.random.default_rng(N + mk + int(causal))
    nqb, nkb = N // 128, N // 64
    B, Hq = (2, 3) if N <= 8192 else (1, 1)
    log(f"patterns: random lists N={N} mk={mk} lines {nv}+{ns} causal={causal}")
    # lists biased toward a few columns and distances, so that lines exist,
    # with duplicates, invalid entries and counts past mk
    idx = rng.integers(-2, nkb + 2, (B, Hq, nqb, mk)).astype(np.int32)
    col = rng.integers(0, nkb, 3)
    for i in range(nqb):
        if rng.random() < 0.6:
            idx[:, :, i, 0] = col[i % 3]
        if rng.random() < 0.6:
            idx[:, :, i, 1] = 2 * i - 5
    idx[:, :, ::7, 2] = idx[:, :, ::7, 3]
    cnt = rng.integers(-1, mk + 3, (B, Hq, nqb)).astype(np.int32)
    p = _P(B, Hq, 1, N, 128, "bf16", causal)
    want = predict_patterns(idx, cnt, N, causal, nv, ns)
    _check(_gpu_patterns(gpu_lib, p, idx, cnt, nv, ns), want)


def test_larger_output_capacity_pads(gpu_lib):
    rng = np.random.default_rng(2)
    N, mk, nv, ns = 2048, 6, 3, 2
    nqb, nkb = N // 128, N // 64
    idx = rng.integers(0, nkb, (1, 2, nqb, mk)).astype(np.int32)
    cnt = np.full((1, 2, nqb), mk, dtype=np.int32)
    p = _P(1, 2, 1, N, 64, "f16", True)
    want = predict_patterns(idx, cnt, N, True, nv, ns, mk_out=nkb)
    _check(_gpu_patterns(gpu_lib, p, idx, cnt, nv, ns, mk_out=nkb), want)


@pytest.mark.parametrize("mask", ["pooled", "lowbit"])
def test_oracle_masks_bit_exact(gpu_lib, mask):
    p, t = make_case(B=1, Hq=8, Hkv=2, N=4096, d=128, dtype="bf16", causal=True, seed=71,
                     k_offset_std=3.0, outliers=4)
    log(f"patterns on the oracle's {mask} mask, N=4096")
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    if mask == "pooled":
        idx, cnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, True, 1, 10)
    else:
        idx, cnt, _, _ = oracle.lowbit_block_mask(t["q"], t["k"], p.Hq, p.Hkv, True, 1, 10,
                                                  k_mean=sq["k_mean"])
    want = predict_patterns(idx, cnt, p.N, True, 8, 8)
    got = _gpu_patterns(gpu_lib, p, idx, cnt, 8, 8)
    _check(got, want)
    added = int(want[2].sum() - cnt.sum())
    log(f"  lines found: vertical {int((want[0][..., :8] >= 0).sum())}, "
        f"slash {int((want[0][..., 8:] > np.iinfo(np.int32).min).sum())}; blocks added {added}")


def test_full_size_pooled_mask_bit_exact(gpu_lib):
    # the block-sparse workload (N = 32768, 32 query heads): the oracle's
    # pooled lists of every head through both predictions
    p, t = make_config(5)
    keep = p.sparse
    log(f"patterns full size: {p.name}, keep {keep}")
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, p.causal,
                                       keep[0], keep[1])
    want = predict_patterns(idx, cnt, p.N, p.causal, 16, 16)
    _check(_gpu_patterns(gpu_lib, p, idx, cnt, 16, 16), want)
    # the chain: the GPU's own mask, then its own prediction; compared on the
    # heads whose lists agree everywhere (the others hold a reported near-tie)
    plan, _ = _chain(gpu_lib, p, t, keep, (16, 16))
    gi, gc = to_np(plan.mask_idx), to_np(plan.mask_cnt)
    agree = same_lists(gi, gc, idx, cnt, ties)
    heads = np.all(agree, axis=-1)
    log(f"  heads with identical masks: {int(heads.sum())} of {heads.size}")
    assert heads.sum() >= heads.size // 2
    gl = to_np(plan.lines)
    for b in range(p.B):
        for h in range(p.Hq):
            if heads[b, h]:
                assert np.array_equal(gl[b, h], want[0][b, h])
                assert np.array_equal(to_np(plan.kv_cnt)[b, h], want[2][b, h])
                assert np.array_equal(to_np(plan.kv_idx)[b, h], want[1][b, h])


def _chain(qa, p, t, keep, patterns):
    q, k, v = (t[x].to(DEV) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), DEV, sparse=keep,
                   with_lse=True, patterns=patterns)
    o = torch.empty_like(q)
    plan.run(q, k, v, o)
    torch.cuda.synchronize()
    return plan, o


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f16", False)])
def test_forward_over_extended_lists(gpu_lib, dtype, causal):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=2048, d=128, dtype=dtype, causal=causal, seed=72,
                     k_offset_std=3.0, outliers=4)
    log(f"sparse forward over pattern-extended lists {dtype} causal={causal}")
    plan, o = _chain(gpu_lib, p, t, (1, 10), (4, 4))
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, causal, 1, 10)
    agree = same_lists(to_np(plan.mask_idx), to_np(plan.mask_cnt), idx, cnt, ties)
    assert np.all(agree), "near-tie in this seeded case"
    lines, eidx, ecnt = predict_patterns(idx, cnt, p.N, causal, 4, 4)
    assert np.array_equal(to_np(plan.kv_idx), eidx) and np.array_equal(to_np(plan.kv_cnt), ecnt)
    assert ecnt.sum() > cnt.sum()       # the lines add blocks
    (_, pre, lse), (_, pre0, _) = emulate_both(
        oracle.emulate_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
        causal, p.Hq, p.Hkv, kv_idx=eidx, kv_cnt=ecnt)
    check_out(to_np(o), pre, pre0, p.dtype, v=t["v"])
    dl = float(np.abs(to_np(plan.lse) - lse).max())
    log(f"  lse_err={dl:.2e}, kept blocks {int(cnt.sum())} -> {int(ecnt.sum())}")
    assert dl < 1e-4
