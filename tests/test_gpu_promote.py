"""GPU parity of the promoted path (qattn_fwd_promoted: the kept blocks at
16-bit Q K^T, every other visible block through the INT8 path) against the
oracle's emulation of it, through the C ABI.

Each side computes its own smoothing, quantization and block mask; the masks
are compared first (bit-exact but for near-ties) and the outputs wherever the
two lists agree. Bars as for qattn_fwd: within TOL_EMU of the emulation (before
its final rounding), lse within 1e-4, cosine >= COS_MIN against exact fp64
attention -- here over every key, since promotion skips nothing.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_case
from parity_util import (TOL_EMU, COS_MIN, KERNEL_TAU, log, out_err, cos, to_np, run_gpu,
                         same_lists, block_rows, emulate_both, check_out)

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16-d128-causal-gqa4-N2048-keep10", dict(B=1, Hq=8, Hkv=2, N=2048, d=128, dtype="bf16",
                                                causal=True, seed=41, k_offset_std=3.0,
                                                outliers=4), (1, 10)),
    ("f16-d64-nc-B2-N640-keep25", dict(B=2, Hq=4, Hkv=4, N=640, d=64, dtype="f16",
                                       causal=False, seed=42, k_offset_std=2.0), (1, 4)),
    ("bf16-d64-causal-mqa-N512-keep25", dict(B=1, Hq=4, Hkv=1, N=512, d=64, dtype="bf16",
                                             causal=True, seed=43, k_offset_std=3.0,
                                             outliers=2), (1, 4)),
    ("f16-d128-causal-N384-forced-only", dict(B=1, Hq=4, Hkv=2, N=384, d=128, dtype="f16",
                                              causal=True, seed=44, k_offset_std=2.0), (0, 1)),
    ("bf16-d128-nc-N512-all", dict(B=1, Hq=2, Hkv=1, N=512, d=128, dtype="bf16", causal=False,
                                   seed=45, k_offset_std=3.0, outliers=4), (1, 1)),
]


def _oracle_promoted(p, t, keep, max_keep):
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, p.causal,
                                       keep[0], keep[1], max_keep)
    (O_emu, O_pre, lse), (_, O_pre0, _) = emulate_both(
        oracle.emulate_promoted_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
        t["q"], t["k"], sq["k_mean"], t["v"], p.causal, p.Hq, p.Hkv, idx, cnt)
    return sq, idx, cnt, ties, O_pre, O_pre0, lse


@pytest.mark.parametrize("name,kw,keep", CASES, ids=[c[0] for c in CASES])
def test_promoted_fwd_matches_emulation(gpu_lib, name, kw, keep):
    p, t = make_case(**kw)
    log(f"promoted fwd {name}")
    plan, o = run_gpu(gpu_lib, p, t, sparse=keep, promote=True)
    sq, idx, cnt, ties, O_pre, O_pre0, lse_emu = _oracle_promoted(p, t, keep, plan.max_keep)
    rows = block_rows(same_lists(to_np(plan.kv_idx), to_np(plan.kv_cnt), idx, cnt, ties))
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], p.causal)
    og = to_np(o)
    check_out(og[rows], O_pre[rows], O_pre0[rows], p.dtype, v=t["v"])
    c = cos(og[rows], O_ex[rows])
    dl = float(np.abs(to_np(plan.lse)[rows] - lse_emu[rows]).max())
    log(f"  lse_err={dl:.2e} cos_exact={c:.6f} rows={rows.mean():.3f}")
    assert dl < 1e-4
    assert c >= COS_MIN


def test_promoted_hand_made_lists(gpu_lib):
    # duplicates, out-of-range and causally invisible entries, counts above
    # max_keep and empty lists: the kernel must promote exactly promote_plan's set
    p, t = make_case(B=1, Hq=2, Hkv=1, N=768, d=128, dtype="bf16", causal=True, seed=46,
                     k_offset_std=3.0, outliers=4)
    log("promoted fwd, hand-made kept lists")
    dev = torch.device("cuda:0")
    qa = gpu_lib
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev, with_lse=True)
    plan.smooth_quant(q, k)
    nqb, nkb, mk = p.N // 128, p.N // 64, 6
    rng = np.random.default_rng(7)
    idx = rng.integers(-2, nkb + 2, (1, 2, nqb, mk)).astype(np.int32)
    idx[0, 0, :, 1] = idx[0, 0, :, 0]                # duplicates
    cnt = rng.integers(0, mk + 3, (1, 2, nqb)).astype(np.int32)  # some above max_keep
    cnt[0, 1, 0] = 0                                  # an empty list
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.N), dtype=torch.float32, device=dev)
    qa.qattn_fwd_promoted(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, torch.from_numpy(idx).to(dev),
                          torch.from_numpy(cnt).to(dev), mk, o, lse)
    torch.cuda.synchronize()
    sq = oracle.smooth_quant(t["q"], t["k"])
    (_, O_pre, lse_emu), (_, O_pre0, _) = emulate_both(
        oracle.emulate_promoted_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
        t["q"], t["k"], sq["k_mean"], t["v"], True, 2, 1, idx, np.minimum(cnt, mk))
    check_out(to_np(o), O_pre, O_pre0, p.dtype, v=t["v"])
    dl = float(np.abs(to_np(lse) - lse_emu).max())
    log(f"  lse_err={dl:.2e}")
    assert dl < 1e-4


def test_promote_nothing_equals_dense_bit_exact(gpu_lib):
    # an empty promoted set leaves the INT8 path, which runs the same
    # arithmetic in the same order as the dense kernel
    p, t = make_case(B=1, Hq=4, Hkv=2, N=1024, d=128, dtype="bf16", causal=True, seed=47,
                     k_offset_std=3.0)
    log("promoted fwd with nothing promoted vs dense")
    dev = torch.device("cuda:0")
    qa = gpu_lib
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan, o_dense = run_gpu(qa, p, t)
    nqb = p.N // 128
    idx = torch.full((1, 4, nqb, 1), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros((1, 4, nqb), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    qa.qattn_fwd_promoted(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, idx, cnt, 1, o, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_promoted_closed_forms(gpu_lib, dtype):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=128, dtype=dtype, causal=True, seed=48,
                     k_offset_std=3.0)
    t1 = dict(t, v=torch.ones_like(t["v"]))
    _, o = run_gpu(gpu_lib, p, t1, sparse=(1, 4), promote=True)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert torch.all((o.double() - 1.0).abs() <= u)
    _, o = run_gpu(gpu_lib, p, t, sparse=(1, 4), promote=True)
    v = t["v"].to("cuda:0")
    for hq in range(4):
        assert torch.equal(o[0, hq, 0], v[0, hq // 2, 0])


def test_promote_beats_skip_on_the_gpu(gpu_lib):
    # the summary's claim on the Llama-shaped law: keeping the other blocks at
    # INT8 instead of skipping them brings the output much closer to exact
    # attention, and promoting the top blocks is no worse than INT8 everywhere
    p, t = make_case(B=1, Hq=8, Hkv=2, N=2048, d=128, dtype="bf16", causal=True, seed=49,
                     k_offset_std=3.0, outliers=4)
    log("promote vs skip vs dense INT8 against exact attention")
    _, o_prom = run_gpu(gpu_lib, p, t, sparse=(1, 10), promote=True)
    _, o_skip = run_gpu(gpu_lib, p, t, sparse=(1, 10))
    _, o_dense = run_gpu(gpu_lib, p, t)
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], True)

    def rms(o):
        return float(np.sqrt(np.mean((to_np(o) - O_ex) ** 2)))

    r_p, r_s, r_d = rms(o_prom), rms(o_skip), rms(o_dense)
    log(f"  rms error: promote {r_p:.3e}  skip {r_s:.3e}  dense INT8 {r_d:.3e}")
    assert r_p < 0.5 * r_s
    assert r_p <= r_d * 1.001
