"""GPU parity of the element-level 4-bit block estimator
(qattn_block_mask_lowbit) against the oracle, through the C ABI.

The MX FP4 products are exact in the matrix core's fp32 accumulation whenever
the shared exponents of the summed groups lie within a few binades of each
other (always the case for these inputs), so the block scores are compared
bit for bit, and with them the kept lists.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.lowbit import lowbit_block_mask
from synthetic import make_case
from parity_util import (TOL_EMU, COS_MIN, KERNEL_TAU, log, out_err, cos, to_np, emulate_both,
                         check_out)

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16-d128-causal-gqa4-N1024-keep10", dict(B=1, Hq=8, Hkv=2, N=1024, d=128, dtype="bf16",
                                                causal=True, seed=81, k_offset_std=3.0,
                                                outliers=4), (1, 10)),
    ("f16-d64-nc-B2-N640-keep25", dict(B=2, Hq=4, Hkv=4, N=640, d=64, dtype="f16",
                                       causal=False, seed=82, k_offset_std=2.0), (1, 4)),
    ("bf16-d64-causal-mqa-N512-keep0", dict(B=1, Hq=4, Hkv=1, N=512, d=64, dtype="bf16",
                                            causal=True, seed=83, k_offset_std=3.0), (0, 1)),
    ("bf16-d128-causal-N4096-keep10", dict(B=1, Hq=4, Hkv=1, N=4096, d=128, dtype="bf16",
                                           causal=True, seed=84, k_offset_std=3.0,
                                           outliers=4), (1, 10)),
]


def _gpu_lowbit(qa, p, t, keep):
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev)
    plan.smooth_quant(q, k)
    nqb, nkb = p.N // 128, p.N // 64
    mk = qa.qattn_max_keep(plan.p, *keep)
    idx = torch.empty((p.B, p.Hq, nqb, mk), dtype=torch.int32, device=dev)
    cnt = torch.empty((p.B, p.Hq, nqb), dtype=torch.int32, device=dev)
    sc = torch.full((p.B, p.Hq, nqb, nkb), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(qa.qattn_lowbit_workspace_bytes(plan.p), dtype=torch.uint8, device=dev)
    qa.qattn_block_mask_lowbit(plan.p, q, k, plan.k_mean, keep[0], keep[1], mk, idx, cnt, sc, ws)
    torch.cuda.synchronize()
    return dev, q, k, v, plan, idx, cnt, sc, mk


@pytest.mark.parametrize("name,kw,keep", CASES, ids=[c[0] for c in CASES])
def test_lowbit_scores_and_mask_bit_exact(gpu_lib, name, kw, keep):
    p, t = make_case(**kw)
    log(f"low-bit mask {name}")
    dev, q, k, v, plan, idx, cnt, sc, mk = _gpu_lowbit(gpu_lib, p, t, keep)
    o_idx, o_cnt, ties, o_sc = lowbit_block_mask(t["q"], t["k"], p.Hq, p.Hkv, p.causal,
                                                 keep[0], keep[1], mk)
    g = to_np(sc)
    valid = np.isfinite(o_sc)
    assert np.array_equal(g[valid], o_sc[valid].astype(np.float32))
    assert np.array_equal(to_np(cnt), o_cnt)
    assert np.array_equal(to_np(idx), o_idx)
    log(f"  scores and lists bit-exact; near-tie rows {int(ties.sum())}")


def test_lowbit_mask_drives_the_sparse_forward(gpu_lib):
    # the kept lists feed qattn_fwd (skip) and qattn_fwd_promoted unchanged;
    # both match their emulations under the oracle's own low-bit lists
    p, t = make_case(B=1, Hq=4, Hkv=2, N=2048, d=128, dtype="bf16", causal=True, seed=85,
                     k_offset_std=3.0, outliers=4)
    qa = gpu_lib
    keep = (1, 10)
    dev, q, k, v, plan, idx, cnt, sc, mk = _gpu_lowbit(qa, p, t, keep)
    o_skip, o_prom = torch.empty_like(q), torch.empty_like(q)
    qa.qattn_fwd(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v, idx, cnt, mk,
                 o_skip, None)
    qa.qattn_fwd_promoted(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, idx, cnt, mk, o_prom, None)
    torch.cuda.synchronize()
    o_idx, o_cnt, _, _ = lowbit_block_mask(t["q"], t["k"], p.Hq, p.Hkv, True, keep[0], keep[1],
                                           mk)
    sq = oracle.smooth_quant(t["q"], t["k"])
    (_, pre_skip, _), (_, pre_skip0, _) = emulate_both(
        oracle.emulate_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
        True, p.Hq, p.Hkv, kv_idx=o_idx, kv_cnt=o_cnt)
    (_, pre_prom, _), (_, pre_prom0, _) = emulate_both(
        oracle.emulate_promoted_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
        t["q"], t["k"], sq["k_mean"], t["v"], True, p.Hq, p.Hkv, o_idx, o_cnt)
    ex_mask, _ = oracle.exact_attention(t["q"], t["k"], t["v"], True, o_idx, o_cnt)
    check_out(to_np(o_skip), pre_skip, pre_skip0, p.dtype, "skip: ", v=t["v"])
    check_out(to_np(o_prom), pre_prom, pre_prom0, p.dtype, "promoted: ", v=t["v"])
    c1 = cos(to_np(o_skip), ex_mask)
    log(f"  skip cos_exact_same_mask={c1:.6f}")
    assert c1 >= COS_MIN


def test_lowbit_finds_a_planted_element_the_pooled_mask_misses(gpu_lib):
    # one large query-key product (q . k = 128 * 1.1^2, about three times the
    # largest product of an ordinary block) inside an otherwise ordinary
    # block: its block means move by about 1 %, its element-level estimate
    # dominates (checked on the oracle for this seed: the pooled mask keeps
    # blocks 11 and 13, the low-bit one 7 and 13)
    p, t = make_case(B=1, Hq=1, Hkv=1, N=2048, d=128, dtype="bf16", causal=True, seed=86,
                     k_offset_std=1.0)
    q, k = t["q"].clone(), t["k"].clone()
    kmean = k[0, 0].float().mean(0)
    q[0, 0, 12 * 128 + 40] = 1.1
    k[0, 0, 7 * 64 + 20] = (1.1 + kmean).to(torch.bfloat16)
    t = dict(t, q=q, k=k)
    qa = gpu_lib
    keep = (1, 16)
    dev, qd, kd, v, plan, idx, cnt, sc, mk = _gpu_lowbit(qa, p, t, keep)
    kept_lowbit = set(to_np(idx)[0, 0, 12, :int(to_np(cnt)[0, 0, 12])].tolist())
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    pidx, pcnt, _ = oracle.block_mask(sq["q_pool"], sq["k_pool"], 1, 1, True, keep[0], keep[1], mk)
    kept_pooled = set(pidx[0, 0, 12, :pcnt[0, 0, 12]].tolist())
    log(f"  block 7 kept: low-bit {7 in kept_lowbit}, pooled {7 in kept_pooled}")
    assert 7 in kept_lowbit
    assert 7 not in kept_pooled
