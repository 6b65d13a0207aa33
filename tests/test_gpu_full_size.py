"""GPU parity at the full sizes of the workloads for the paths the benchmark
times besides the dense and block-sparse forwards: the promoted forward with
its INT8 and its MX FP4 low path (the Llama-shaped causal N = 8192 workload and
the block-sparse N = 32768 one), the per-head error proxy and the adaptive
forward (N = 8192), and the element-level 4-bit block mask (N = 32768). Same
bars as the small cases; each side computes its own smoothing, quantization
and lists, which are compared first.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.lowbit import lowbit_block_mask
from synthetic import make_config
from parity_util import (COS_MIN, log, cos, to_np, run_gpu, head_slice, same_lists, emulate_both,
                         check_out)

pytestmark = pytest.mark.gpu

COS_MIN_FP4 = 0.98
ADAPTIVE_THRESHOLD = 0.019  # the benchmark's setting at N = 8192: splits the heads of that law

def _slices(p):
    """(b, kv head, query heads) of the first kv head of the first batch entry
    and the last of the last, two query heads each (the group's ends)."""
    out = []
    for b, hk in sorted({(0, 0), (p.B - 1, p.Hkv - 1)}):
        hqs = [hk * p.group, hk * p.group + p.group - 1] if p.group > 1 else [hk]
        out.append((b, hk, hqs))
    return out

@pytest.mark.parametrize("low4", [False, True], ids=["int8-low", "fp4-low"])
@pytest.mark.parametrize("c", [2, 5])
def test_promoted_full_size_sampled(gpu_lib, c, low4):
    p, t = make_config(c)
    keep = p.sparse if p.sparse is not None else (1, 10)
    log(f"promoted full size ({'MX FP4' if low4 else 'INT8'} low path): {p.name}, keep {keep}")
    plan, o = run_gpu(gpu_lib, p, t, sparse=keep, pools=True, promote=True, low4=low4)
    nqb = p.N // 128
    for b, hk, hqs in _slices(p):
        sub, _ = head_slice(t, p, b, hqs)
        ref = oracle.smooth_quant(sub["q"], sub["k"], pools=True)
        idx, cnt, ties = oracle.block_mask(ref["q_pool"], ref["k_pool"], len(hqs), 1, p.causal,
                                           keep[0], keep[1], plan.max_keep)
        agree = same_lists(to_np(plan.kv_idx)[b, hqs][None], to_np(plan.kv_cnt)[b, hqs][None],
                           idx, cnt, ties)
        sel = [(0, n, i) for n in range(len(hqs)) for i in (0, nqb // 2, nqb - 1)
               if agree[0, n, i]]
        blocks = sorted({i for (_, _, i) in sel})
        if low4:
            (_, pre, _), (_, pre0, _) = emulate_both(
                oracle.emulate_promoted_fp4_attention, sub["q"], sub["k"], ref["k_mean"],
                sub["v"], p.causal, len(hqs), 1, idx, cnt, blocks=sel)
        else:
            (_, pre, _), (_, pre0, _) = emulate_both(
                oracle.emulate_promoted_attention, ref["q_i8"], ref["q_scale"], ref["k_i8"],
                ref["k_scale"], sub["q"], sub["k"], ref["k_mean"], sub["v"], p.causal, len(hqs),
                1, idx, cnt, blocks=sel)
        ex, _ = oracle.exact_attention(sub["q"], sub["k"], sub["v"], p.causal, blocks=sel)
        rows = np.concatenate([np.arange(i * 128, i * 128 + 128) for i in blocks])
        g = to_np(o[b, hqs])[None][:, :, rows]
        check_out(g, pre[:, :, rows], pre0[:, :, rows], p.dtype,
                  f"b{b} kv head {hk}, {len(sel)} blocks: ", v=sub["v"])
        cc = cos(g, ex[:, :, rows])
        log(f"  cos_exact={cc:.6f}")
        # the 4-bit low path's Q K^T error is that of 4-bit codes
        assert cc >= (COS_MIN_FP4 if low4 else COS_MIN)

def _adaptive_gpu(qa, p, t):
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev, with_lse=True)
    plan.smooth_quant(q, k)
    err = torch.empty((p.B, p.Hq), dtype=torch.float32, device=dev)
    hi = torch.empty((p.B, p.Hq), dtype=torch.int32, device=dev)
    qa.qattn_head_error(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                        plan.k_mean, ADAPTIVE_THRESHOLD, err, hi)
    o = torch.empty_like(q)
    qa.qattn_fwd_adaptive(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, hi, o, plan.lse)
    torch.cuda.synchronize()
    return plan, err, hi, o

def test_head_error_and_adaptive_full_size_n8192(gpu_lib):
    p, t = make_config(2)
    log(f"head error + adaptive full size: {p.name}, threshold {ADAPTIVE_THRESHOLD}")
    plan, err, hi, o = _adaptive_gpu(gpu_lib, p, t)
    # the error of every head against the oracle's fp64 value
    sq = oracle.smooth_quant(t["q"], t["k"])
    e = oracle.head_error(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["q"], t["k"],
                          sq["k_mean"], p.Hq, p.Hkv)
    g = to_np(err).astype(np.float64)
    rel = float(np.abs(g - e).max() / e.max())
    flags = e > ADAPTIVE_THRESHOLD
    near = np.abs(e - ADAPTIVE_THRESHOLD) <= 1e-4 * ADAPTIVE_THRESHOLD
    log(f"  {p.Hq} heads: errors {e.min():.4f}-{e.max():.4f}, max rel diff {rel:.2e}, "
        f"flagged {int(flags.sum())}, near-ties {int(near.sum())}")
    assert rel < 1e-4
    gflags = to_np(hi) != 0
    assert np.array_equal(gflags[~near], flags[~near])
    # the adaptive forward on sampled blocks of a flagged and an unflagged head
    # (where the group has them) of the first and the last kv head
    nqb = p.N // 128
    for b, hk, _ in _slices(p):
        group = range(hk * p.group, (hk + 1) * p.group)
        ok = [h for h in group if gflags[b, h] == flags[b, h] and not near[b, h]]
        hqs = sorted({next((h for h in ok if flags[b, h]), ok[0]),
                      next((h for h in ok if not flags[b, h]), ok[-1])})
        sub, _ = head_slice(t, p, b, hqs)
        ref = oracle.smooth_quant(sub["q"], sub["k"])
        idx, cnt = oracle.adaptive_lists(flags[b, hqs][None], p.N, p.causal)
        sel = [(0, n, i) for n in range(len(hqs)) for i in (0, nqb // 2, nqb - 1)]
        (_, pre, _), (_, pre0, _) = emulate_both(
            oracle.emulate_promoted_attention, ref["q_i8"], ref["q_scale"], ref["k_i8"],
            ref["k_scale"], sub["q"], sub["k"], ref["k_mean"], sub["v"], p.causal, len(hqs), 1,
            idx, cnt, blocks=sel)
        ex, _ = oracle.exact_attention(sub["q"], sub["k"], sub["v"], p.causal, blocks=sel)
        rows = np.concatenate([np.arange(i * 128, i * 128 + 128) for i in (0, nqb // 2, nqb - 1)])
        g = to_np(o[b, hqs])[None][:, :, rows]
        check_out(g, pre[:, :, rows], pre0[:, :, rows], p.dtype,
                  f"b{b} kv head {hk} heads {hqs} (16-bit {flags[b, hqs].tolist()}): ",
                  v=sub["v"])
        cc = cos(g, ex[:, :, rows])
        log(f"  cos_exact={cc:.6f}")
        assert cc >= COS_MIN

def test_lowbit_mask_full_size_n32768(gpu_lib):
    # the block-sparse workload (N = 32768): scores and kept lists of two query
    # heads, every query block, bit for bit
    qa = gpu_lib
    p, t = make_config(5)
    keep = p.sparse
    log(f"low-bit mask full size: {p.name}, keep {keep}")
    dev = torch.device("cuda:0")
    q, k = t["q"].to(dev), t["k"].to(dev)
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
    hk = p.Hkv - 1
    hqs = [hk * p.group, hk * p.group + p.group - 1]
    sub, _ = head_slice(t, p, 0, hqs)
    o_idx, o_cnt, ties, o_sc = lowbit_block_mask(sub["q"], sub["k"], len(hqs), 1, p.causal,
                                                 keep[0], keep[1], mk)
    g = to_np(sc)[0, hqs][None]
    valid = np.isfinite(o_sc)
    assert np.array_equal(g[valid], o_sc[valid].astype(np.float32))
    assert np.array_equal(to_np(cnt)[0, hqs][None], o_cnt)
    assert np.array_equal(to_np(idx)[0, hqs][None], o_idx)
    log(f"  2 heads x {nqb} query blocks: scores and lists bit-exact "
        f"({int(valid.sum())} scores, near-tie rows {int(ties.sum())})")
