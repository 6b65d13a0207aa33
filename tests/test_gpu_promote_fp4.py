"""GPU parity of promote instead of skip with the MX FP4 low path
(qattn_fwd_promoted_fp4: the kept blocks at 16-bit Q K^T, every other visible
block at MX FP4 Q K^T) against the oracle's emulation of it, through the C ABI.

Each side computes its own smoothing, block mask and MX FP4 codes; the masks
are compared first (bit-exact but for near-ties) and the outputs wherever the
two lists agree. Bars as for qattn_fwd_promoted: within TOL_EMU of the
emulation (before its final rounding), lse within 1e-4; against exact fp64
attention the 4-bit low path keeps the cosine above 0.98 (its Q K^T error is
that of 4-bit codes, far above the INT8 path's).
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_case
from parity_util import (KERNEL_TAU, log, cos, to_np, run_gpu, same_lists, block_rows,
                         emulate_both, check_out)

pytestmark = pytest.mark.gpu

COS_MIN_FP4 = 0.98

CASES = [
    ("bf16-d128-causal-gqa4-N2048-keep10", dict(B=1, Hq=8, Hkv=2, N=2048, d=128, dtype="bf16",
                                                causal=True, seed=61, k_offset_std=3.0,
                                                outliers=4), (1, 10)),
    ("f16-d64-nc-B2-N640-keep25", dict(B=2, Hq=4, Hkv=4, N=640, d=64, dtype="f16",
                                       causal=False, seed=62, k_offset_std=2.0), (1, 4)),
    ("bf16-d64-causal-mqa-N512-keep25", dict(B=1, Hq=4, Hkv=1, N=512, d=64, dtype="bf16",
                                             causal=True, seed=63, k_offset_std=3.0,
                                             outliers=2), (1, 4)),
    ("f16-d128-causal-N384-forced-only", dict(B=1, Hq=4, Hkv=2, N=384, d=128, dtype="f16",
                                              causal=True, seed=64, k_offset_std=2.0), (0, 1)),
    ("bf16-d128-nc-N1152-keep10", dict(B=1, Hq=2, Hkv=1, N=1152, d=128, dtype="bf16",
                                       causal=False, seed=65, k_offset_std=3.0, outliers=4),
     (1, 10)),
    ("bf16-d64-causal-group3-B2-N768-keep10", dict(B=2, Hq=6, Hkv=2, N=768, d=64,
                                                   dtype="bf16", causal=True, seed=60,
                                                   k_offset_std=3.0, outliers=2), (1, 10)),
]


def _oracle_fp4(p, t, keep, max_keep):
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, p.causal,
                                       keep[0], keep[1], max_keep)
    (_, O_pre, lse), (_, O_pre0, _) = emulate_both(
        oracle.emulate_promoted_fp4_attention, t["q"], t["k"], sq["k_mean"], t["v"], p.causal,
        p.Hq, p.Hkv, idx, cnt)
    return sq, idx, cnt, ties, O_pre, O_pre0, lse


def _fwd_fp4(qa, plan, q, k, v, idx, cnt, max_keep, with_lse=True):
    dev = q.device
    o = torch.empty_like(q)
    lse = (torch.empty((plan.p.B, plan.p.Hq, plan.p.N), dtype=torch.float32, device=dev)
           if with_lse else None)
    ws = torch.empty(qa.qattn_lowbit_workspace_bytes(plan.p), dtype=torch.uint8, device=dev)
    qa.qattn_fwd_promoted_fp4(plan.p, q, k, plan.k_mean, v, idx, cnt, max_keep, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("name,kw,keep", CASES, ids=[c[0] for c in CASES])
def test_fp4_promoted_fwd_matches_emulation(gpu_lib, name, kw, keep):
    p, t = make_case(**kw)
    log(f"promoted fwd, MX FP4 low path {name}")
    plan, o = run_gpu(gpu_lib, p, t, sparse=keep, promote=True, low4=True)
    sq, idx, cnt, ties, O_pre, O_pre0, lse_emu = _oracle_fp4(p, t, keep, plan.max_keep)
    rows = block_rows(same_lists(to_np(plan.kv_idx), to_np(plan.kv_cnt), idx, cnt, ties))
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], p.causal)
    og = to_np(o)
    check_out(og[rows], O_pre[rows], O_pre0[rows], p.dtype, v=t["v"])
    c = cos(og[rows], O_ex[rows])
    dl = float(np.abs(to_np(plan.lse)[rows] - lse_emu[rows]).max())
    log(f"  lse_err={dl:.2e} cos_exact={c:.6f} rows={rows.mean():.3f}")
    assert dl < 1e-4
    assert c >= COS_MIN_FP4


def test_fp4_hand_made_lists(gpu_lib):
    # duplicates, out-of-range and causally invisible entries, counts above
    # max_keep and empty lists: the kernel must promote exactly promote_plan's
    # set and take every other visible tile at 4 bits
    p, t = make_case(B=1, Hq=2, Hkv=1, N=768, d=128, dtype="bf16", causal=True, seed=66,
                     k_offset_std=3.0, outliers=4)
    log("promoted fwd (MX FP4 low path), hand-made kept lists")
    dev = torch.device("cuda:0")
    qa = gpu_lib
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev)
    plan.smooth_quant(q, k)
    nqb, nkb, mk = p.N // 128, p.N // 64, 6
    rng = np.random.default_rng(8)
    idx = rng.integers(-2, nkb + 2, (1, 2, nqb, mk)).astype(np.int32)
    idx[0, 0, :, 1] = idx[0, 0, :, 0]                # duplicates
    cnt = rng.integers(0, mk + 3, (1, 2, nqb)).astype(np.int32)  # some above max_keep
    cnt[0, 1, 0] = 0                                  # an empty list
    o, lse = _fwd_fp4(qa, plan, q, k, v, torch.from_numpy(idx).to(dev),
                      torch.from_numpy(cnt).to(dev), mk)
    sq = oracle.smooth_quant(t["q"], t["k"])
    (_, O_pre, lse_emu), (_, O_pre0, _) = emulate_both(
        oracle.emulate_promoted_fp4_attention, t["q"], t["k"], sq["k_mean"], t["v"], True, 2, 1,
        idx, np.minimum(cnt, mk))
    check_out(to_np(o), O_pre, O_pre0, p.dtype, v=t["v"])
    dl = float(np.abs(to_np(lse) - lse_emu).max())
    log(f"  lse_err={dl:.2e}")
    assert dl < 1e-4


def test_fp4_everything_promoted_equals_int8_variant_bit_exact(gpu_lib):
    # no low tile: the promoted halves run the same arithmetic in the same
    # order whichever low path the call has
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=128, dtype="bf16", causal=False, seed=67,
                     k_offset_std=3.0)
    log("MX FP4 low path with everything promoted vs the INT8-low variant")
    plan4, o4 = run_gpu(gpu_lib, p, t, sparse=(1, 1), promote=True, low4=True)
    plan8, o8 = run_gpu(gpu_lib, p, t, sparse=(1, 1), promote=True)
    assert torch.equal(plan4.kv_cnt, plan8.kv_cnt)
    assert int(plan4.kv_cnt.min()) == p.N // 64
    assert torch.equal(o4, o8)
    assert torch.equal(plan4.lse, plan8.lse)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp4_closed_forms(gpu_lib, dtype):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=128, dtype=dtype, causal=True, seed=68,
                     k_offset_std=3.0)
    t1 = dict(t, v=torch.ones_like(t["v"]))
    _, o = run_gpu(gpu_lib, p, t1, sparse=(1, 4), promote=True, low4=True)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert torch.all((o.double() - 1.0).abs() <= u)
    _, o = run_gpu(gpu_lib, p, t, sparse=(1, 4), promote=True, low4=True)
    v = t["v"].to("cuda:0")
    for hq in range(4):
        assert torch.equal(o[0, hq, 0], v[0, hq // 2, 0])


def test_fp4_low_path_between_skip_and_int8_on_the_gpu(gpu_lib):
    # on the Llama-shaped law: keeping the other blocks at 4 bits is much
    # closer to exact attention than skipping them, and no closer than
    # keeping them at INT8
    p, t = make_case(B=1, Hq=8, Hkv=2, N=2048, d=128, dtype="bf16", causal=True, seed=69,
                     k_offset_std=3.0, outliers=4)
    log("promote (MX FP4 low) vs promote (INT8 low) vs skip against exact attention")
    _, o4 = run_gpu(gpu_lib, p, t, sparse=(1, 10), promote=True, low4=True)
    _, o8 = run_gpu(gpu_lib, p, t, sparse=(1, 10), promote=True)
    _, o_skip = run_gpu(gpu_lib, p, t, sparse=(1, 10))
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], True)

    def rms(o):
        return float(np.sqrt(np.mean((to_np(o) - O_ex) ** 2)))

    r4, r8, rs = rms(o4), rms(o8), rms(o_skip)
    log(f"  rms error: promote/fp4 {r4:.3e}  promote/int8 {r8:.3e}  skip {rs:.3e}")
    assert r4 < 0.5 * rs
    assert r8 <= r4
