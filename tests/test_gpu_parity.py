"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: smoothing/quantization outputs (codes, scales, channel means, pooled
means) and the block mask are bit-exact (mask rows at a near-tie excepted); the
attention output is within TOL_EMU of the quantized-path emulation (before the
final 16-bit rounding, see parity_util.out_err) and has cosine >= COS_MIN
against exact fp64 attention (under the same block mask when sparse).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_case, make_config
from parity_util import (TOL_EMU, COS_MIN, KERNEL_TAU, log, out_err, max_abs_rel, cos, to_np,
                         run_gpu, head_slice, same_lists, block_rows, emulate_both, check_out)

pytestmark = pytest.mark.gpu

# (name, make_case kwargs): several 64/128-row tiles, GQA on/off, both dtypes,
# both head sizes, N not a power of two (a partial K-sum chunk, N/128 odd)
SMALL = [
    ("c1", None),
    ("bf16-d128-causal-gqa4-N1024", dict(B=1, Hq=8, Hkv=2, N=1024, d=128, dtype="bf16",
                                         causal=True, seed=21, k_offset_std=3.0, outliers=4)),
    ("f16-d64-nc-B2-N640", dict(B=2, Hq=4, Hkv=4, N=640, d=64, dtype="f16", causal=False,
                                seed=22, k_offset_std=2.0)),
    ("f16-d128-causal-gqa2-N384", dict(B=1, Hq=4, Hkv=2, N=384, d=128, dtype="f16",
                                       causal=True, seed=23, k_offset_std=2.0)),
    ("bf16-d64-causal-mqa-N512", dict(B=1, Hq=4, Hkv=1, N=512, d=64, dtype="bf16",
                                      causal=True, seed=24, k_offset_std=3.0, outliers=2)),
    # three query heads per kv head: the dense layout takes one head per
    # 8-wave workgroup (256 rows) instead of 4 heads x 2 slabs
    ("f16-d128-causal-group3-N768", dict(B=2, Hq=6, Hkv=2, N=768, d=128, dtype="f16",
                                         causal=True, seed=25, k_offset_std=3.0, outliers=2)),
    # d = 64 dense runs 4-wave workgroups: two query heads x 64 rows (group 2)
    # and one head x 128 rows (group 3, causal, N/128 odd)
    ("bf16-d64-causal-gqa2-N384", dict(B=1, Hq=4, Hkv=2, N=384, d=64, dtype="bf16",
                                       causal=True, seed=26, k_offset_std=3.0, outliers=2)),
    ("f16-d64-causal-group3-N640", dict(B=1, Hq=6, Hkv=2, N=640, d=64, dtype="f16",
                                        causal=True, seed=27, k_offset_std=2.0)),
    # the shortest sequences the library takes (one 128-row query block, two
    # key tiles): most waves of a workgroup have no rows
    ("f16-d64-causal-N128", dict(B=1, Hq=2, Hkv=1, N=128, d=64, dtype="f16", causal=True,
                                 seed=28, k_offset_std=2.0)),
    ("bf16-d128-nc-mqa4-N128", dict(B=1, Hq=4, Hkv=1, N=128, d=128, dtype="bf16",
                                    causal=False, seed=29, k_offset_std=3.0, outliers=2)),
]


def _case(name, kw):
    if kw is None:
        return make_config(1)
    return make_case(**kw)


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_smooth_quant_bit_exact(gpu_lib, name, kw):
    p, t = _case(name, kw)
    log(f"smooth_quant {name}")
    plan, _ = run_gpu(gpu_lib, p, t, pools=True)
    ref = oracle.smooth_quant(t["q"], t["k"], pools=True)
    for key in ["k_mean", "q_scale", "k_scale", "q_pool", "k_pool", "q_i8", "k_i8"]:
        got = to_np(getattr(plan, key))
        want = ref[key]
        assert got.shape == want.shape, key
        bad = np.count_nonzero(got != want)
        assert bad == 0, f"{key}: {bad} of {got.size} differ"


def _tie_blocks(gen, rows, nblk, d, dtype):
    """[nblk*rows, d] values on exact rounding ties: every block holds half-integer
    multiples of a power of two 2^e (and one entry 127 * 2^e, so the block scale is
    exactly 2^e), so x / scale lands on n + 1/2 for most entries."""
    n = torch.randint(-127, 127, (nblk, rows, d), generator=gen).double()
    n = n + 0.5 * torch.randint(0, 2, (nblk, rows, d), generator=gen).double()
    n[:, 0, 0] = 127.0
    e = torch.randint(-6, 4, (nblk, 1, 1), generator=gen).double()
    return (n * torch.exp2(e)).reshape(nblk * rows, d).to(dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_smooth_quant_exact_ties(gpu_lib, dtype, d):
    """Round-half-to-even of the exact quotient on inputs built to sit on ties.
    K is mirrored (second half = minus the first) so its channel mean is exactly
    zero and the smoothing leaves the ties in place."""
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=d, dtype=dtype, causal=True, seed=31)
    tdt = t["q"].dtype
    gen = torch.Generator().manual_seed(31)
    t["q"] = torch.stack([_tie_blocks(gen, 128, p.N // 128, d, tdt) for _ in range(p.Hq)])[None]
    half = _tie_blocks(gen, 64, p.N // 128, d, tdt)
    t["k"] = torch.cat([half, -half])[None, None].contiguous()
    log(f"smooth_quant ties {dtype} d{d}")
    plan, _ = run_gpu(gpu_lib, p, t, pools=True)
    ref = oracle.smooth_quant(t["q"], t["k"], pools=True)
    assert np.all(ref["k_mean"] == 0.0)
    ties = np.count_nonzero(np.abs(np.abs(ref["q_i8"]).astype(np.int32) % 2) == 0)
    assert ties > 0
    for key in ["k_mean", "q_scale", "k_scale", "q_pool", "k_pool", "q_i8", "k_i8"]:
        got = to_np(getattr(plan, key))
        bad = np.count_nonzero(got != ref[key])
        assert bad == 0, f"{key}: {bad} of {got.size} differ"


def test_smooth_quant_wide_range_bf16(gpu_lib):
    """bf16 K and Q whose magnitudes span 2^-61 .. 2^1 within every channel (a
    ratio of 2^62, inside the 2^64 the header states for exact sums): the
    channel means, pooled means, scales and codes are still bit-exact against
    the oracle's math.fsum sums, which need the double-double's low word
    (62 binades do not fit the 53 bits of one double)."""
    p, t = make_case(B=1, Hq=2, Hkv=1, N=1024, d=64, dtype="bf16", causal=True, seed=33)
    gen = torch.Generator().manual_seed(33)

    def wide(shape):
        e = torch.randint(-61, 1, shape, generator=gen).double()
        m = 1.0 + torch.randint(0, 128, shape, generator=gen).double() / 128.0
        sgn = torch.where(torch.rand(shape, generator=gen) < 0.5, -1.0, 1.0).double()
        return (sgn * m * torch.exp2(e)).to(torch.bfloat16)

    t["q"] = wide((1, p.Hq, p.N, p.d)).contiguous()
    t["k"] = wide((1, p.Hkv, p.N, p.d)).contiguous()
    a = t["k"][0, 0].double().abs()
    for c in range(p.d):
        nz = a[:, c][a[:, c] > 0]
        assert float(nz.max() / nz.min()) < 2.0 ** 64
    log("smooth_quant wide-range bf16")
    plan, _ = run_gpu(gpu_lib, p, t, pools=True)
    ref = oracle.smooth_quant(t["q"], t["k"], pools=True)
    for key in ["k_mean", "q_scale", "k_scale", "q_pool", "k_pool", "q_i8", "k_i8"]:
        got = to_np(getattr(plan, key))
        bad = np.count_nonzero(got != ref[key])
        assert bad == 0, f"{key}: {bad} of {got.size} differ"


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_fwd_matches_emulation_and_exact(gpu_lib, name, kw):
    p, t = _case(name, kw)
    log(f"fwd {name}")
    plan, o = run_gpu(gpu_lib, p, t)
    sq = oracle.smooth_quant(t["q"], t["k"])
    (O_emu, O_pre, lse_emu), (_, O_pre0, _) = emulate_both(
        oracle.emulate_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
        p.causal, p.Hq, p.Hkv)
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], p.causal)
    og = to_np(o)
    check_out(og, O_pre, O_pre0, p.dtype, v=t["v"])
    c = cos(og, O_ex)
    log(f"  maxabsrel_rounded={max_abs_rel(og, O_emu):.3e} cos_exact={c:.6f}")
    assert c >= COS_MIN
    lse = to_np(plan.lse)
    assert np.abs(lse - lse_emu).max() < 1e-4


@pytest.mark.parametrize("sparse", [(1, 10), (1, 4), (0, 1), (1, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_block_mask_matches_oracle(gpu_lib, sparse, causal):
    p, t = make_case(B=1, Hq=8, Hkv=2, N=4096, d=128, dtype="bf16", causal=causal, seed=31,
                     k_offset_std=3.0, outliers=4)
    log(f"block_mask causal={causal} keep={sparse}")
    plan, o = run_gpu(gpu_lib, p, t, sparse=sparse)
    ref = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(ref["q_pool"], ref["k_pool"], p.Hq, p.Hkv, causal,
                                       sparse[0], sparse[1], plan.max_keep)
    gi, gc = to_np(plan.kv_idx), to_np(plan.kv_cnt)
    ok = ~ties
    assert np.array_equal(gc[ok], cnt[ok])
    assert np.array_equal(gi[ok], idx[ok])
    # near-tie rows may swap one block; everything else about them is fixed
    assert np.array_equal(gc, cnt)


def test_sparse_fwd_matches_emulation(gpu_lib):
    p, t = make_case(B=1, Hq=8, Hkv=2, N=2048, d=128, dtype="bf16", causal=True, seed=32,
                     k_offset_std=3.0, outliers=4, sparse=(1, 10))
    log("sparse fwd N=2048")
    plan, o = run_gpu(gpu_lib, p, t, sparse=(1, 10))
    # each side uses its own mask; outputs are compared where the lists agree
    sq = oracle.smooth_quant(t["q"], t["k"], pools=True)
    idx, cnt, ties = oracle.block_mask(sq["q_pool"], sq["k_pool"], p.Hq, p.Hkv, True, 1, 10,
                                       plan.max_keep)
    rows = block_rows(same_lists(to_np(plan.kv_idx), to_np(plan.kv_cnt), idx, cnt, ties))
    (_, O_pre, _), (_, O_pre0, _) = emulate_both(
        oracle.emulate_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
        True, p.Hq, p.Hkv, kv_idx=idx, kv_cnt=cnt)
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], True, idx, cnt)
    og = to_np(o)
    check_out(og[rows], O_pre[rows], O_pre0[rows], p.dtype, v=t["v"])
    c = cos(og[rows], O_ex[rows])
    log(f"  cos_exact_same_mask={c:.6f} rows={rows.mean():.3f}")
    assert c >= COS_MIN


def test_sparse_fwd_empty_and_invalid_lists(gpu_lib):
    # kept lists with no usable entry (count 0, or only entries out of range or
    # past the causal range) give O = 0 and lse = -inf; a list of duplicates of
    # one block equals that block alone
    p, t = make_case(B=1, Hq=2, Hkv=1, N=512, d=64, dtype="bf16", causal=True, seed=36)
    log("sparse fwd, empty / invalid / duplicate kept lists")
    dev = torch.device("cuda:0")
    qa = gpu_lib
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev, with_lse=True)
    plan.smooth_quant(q, k)
    nqb, mk = p.N // 128, 4
    idx = torch.full((1, 2, nqb, mk), -1, dtype=torch.int32)
    cnt = torch.zeros((1, 2, nqb), dtype=torch.int32)
    # head 0: count 0 everywhere; head 1, block i: entries -1, 8 (out of range),
    # 2i + 2 (past the causal range when in range), count 3
    for i in range(nqb):
        idx[0, 1, i, :3] = torch.tensor([-1, 8, 2 * i + 2])
        cnt[0, 1, i] = 3
    o = torch.full_like(q, 7.0)
    lse = torch.zeros((1, 2, p.N), dtype=torch.float32, device=dev)
    qa.qattn_fwd(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v,
                 idx.to(dev), cnt.to(dev), mk, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert torch.all(torch.isneginf(lse))
    # duplicates of block 0 (visible to every row) = block 0 once
    idx_dup = torch.zeros((1, 2, nqb, mk), dtype=torch.int32)
    cnt_dup = torch.full((1, 2, nqb), mk, dtype=torch.int32)
    idx_one = torch.zeros((1, 2, nqb, mk), dtype=torch.int32)
    cnt_one = torch.ones((1, 2, nqb), dtype=torch.int32)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    qa.qattn_fwd(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v,
                 idx_one.to(dev), cnt_one.to(dev), mk, o1, None)
    qa.qattn_fwd(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v,
                 idx_dup.to(dev), cnt_dup.to(dev), mk, o2, None)
    torch.cuda.synchronize()
    sq = oracle.smooth_quant(t["q"], t["k"])
    (_, O_pre, _), (_, O_pre0, _) = emulate_both(
        oracle.emulate_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["v"],
        True, 2, 1, kv_idx=idx_one.numpy(), kv_cnt=cnt_one.numpy())
    check_out(to_np(o1), O_pre, O_pre0, p.dtype, "block 0 alone: ", v=t["v"])
    check_out(to_np(o2), O_pre, O_pre0, p.dtype, "block 0 repeated: ", v=t["v"])


def test_keep_all_mask_equals_dense_bit_exact(gpu_lib):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=1024, d=128, dtype="bf16", causal=True, seed=33,
                     k_offset_std=3.0)
    _, o_dense = run_gpu(gpu_lib, p, t)
    _, o_sparse = run_gpu(gpu_lib, p, t, sparse=(1, 1))
    assert torch.equal(o_dense, o_sparse)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_closed_forms_v_ones_and_causal_row0(gpu_lib, dtype):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=128, dtype=dtype, causal=True, seed=34,
                     k_offset_std=3.0)
    # V = 1: O = sum(P_hat) / sum(P), within the unit roundoff u of the 16-bit
    # type of 1 (a dropped or doubled rescale of acc or l breaks this by far)
    t1 = dict(t, v=torch.ones_like(t["v"]))
    _, o = run_gpu(gpu_lib, p, t1)
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert torch.all((o.double() - 1.0).abs() <= u)
    _, o = run_gpu(gpu_lib, p, t)
    v = t["v"].to("cuda:0")
    for hq in range(4):
        assert torch.equal(o[0, hq, 0], v[0, hq // 2, 0])


def test_deterministic_and_no_stray_writes(gpu_lib):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=1024, d=64, dtype="bf16", causal=True, seed=35)
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    qa = gpu_lib
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev,
                   sparse=(1, 10), with_lse=True)
    guard = 4096
    buf = torch.full((q.numel() + 2 * guard,), 12345.0, dtype=q.dtype, device=dev)
    o = buf[guard:guard + q.numel()].view_as(q)
    plan.run(q, k, v, o)
    first = o.clone()
    idx1 = plan.kv_idx.clone()
    plan.run(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.equal(first, o)
    assert torch.equal(idx1, plan.kv_idx)
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[-guard:] == 12345.0)


# ---- the five workloads at full size, compared on sampled heads/blocks ------------

def _sampled_check(qa, c, n_blocks=3):
    p, t = make_config(c)
    log(f"config {c}: {p.name}")
    sparse = p.sparse
    plan, o = run_gpu(qa, p, t, sparse=sparse, pools=True)
    # the first kv head of the first batch entry and the last of the last
    for b, hk in sorted({(0, 0), (p.B - 1, p.Hkv - 1)}):
        _sampled_head(p, t, plan, o, b, hk, n_blocks)


def _sampled_head(p, t, plan, o, b, hk, n_blocks):
    sparse = p.sparse
    hqs = [hk * p.group, hk * p.group + p.group - 1] if p.group > 1 else [hk]
    sub, _ = head_slice(t, p, b, hqs)
    ps = dataclasses.replace(p, B=1, Hq=len(hqs), Hkv=1)
    ref = oracle.smooth_quant(sub["q"], sub["k"], pools=sparse is not None)
    # bit-exact pre-processing on the slice
    assert np.array_equal(to_np(plan.k_mean)[b, hk], ref["k_mean"][0, 0])
    assert np.array_equal(to_np(plan.k_scale)[b, hk], ref["k_scale"][0, 0])
    assert np.array_equal(to_np(plan.k_i8[b, hk]), ref["k_i8"][0, 0])
    for n, hq in enumerate(hqs):
        assert np.array_equal(to_np(plan.q_scale)[b, hq], ref["q_scale"][0, n])
        assert np.array_equal(to_np(plan.q_i8[b, hq]), ref["q_i8"][0, n])
    nqb = p.N // 128
    blocks = sorted({0, nqb // 2, nqb - 1})[:n_blocks]
    sel = [(0, n, i) for n in range(len(hqs)) for i in blocks]
    kv_idx = kv_cnt = None
    if sparse is not None:
        assert np.array_equal(to_np(plan.q_pool)[b, hqs], ref["q_pool"][0])
        assert np.array_equal(to_np(plan.k_pool)[b, hk], ref["k_pool"][0, 0])
        idx, cnt, ties = oracle.block_mask(ref["q_pool"], ref["k_pool"], len(hqs), 1, p.causal,
                                           sparse[0], sparse[1], plan.max_keep)
        gi = to_np(plan.kv_idx)[b, hqs]
        gc = to_np(plan.kv_cnt)[b, hqs]
        agree = same_lists(gi[None], gc[None], idx, cnt, ties)
        # compare only the sampled blocks whose lists agree (all but near-ties)
        sel = [(0, n, i) for (_, n, i) in sel if agree[0, n, i]]
        blocks = sorted({i for (_, _, i) in sel})
        kv_idx, kv_cnt = idx, cnt
    (_, O_pre, _), (_, O_pre0, _) = emulate_both(
        oracle.emulate_attention, ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
        sub["v"], p.causal, ps.Hq, 1, kv_idx=kv_idx, kv_cnt=kv_cnt, blocks=sel)
    O_ex, _ = oracle.exact_attention(sub["q"], sub["k"], sub["v"], p.causal, kv_idx, kv_cnt,
                                     blocks=sel)
    og = to_np(o[b, hqs])[None]
    rows = np.concatenate([np.arange(i * 128, i * 128 + 128) for i in blocks])
    g = og[:, :, rows]
    check_out(g, O_pre[:, :, rows], O_pre0[:, :, rows], p.dtype,
              f"b{b} kv head {hk} sampled {len(sel)} blocks: ", v=sub["v"])
    cc = cos(g, O_ex[:, :, rows])
    log(f"  cos_exact={cc:.6f}")
    assert cc >= COS_MIN


@pytest.mark.parametrize("c", [2, 3, 5])
def test_workload_full_size_sampled(gpu_lib, c):
    _sampled_check(gpu_lib, c)


def test_workload_c4_full_size_sampled(gpu_lib):
    _sampled_check(gpu_lib, 4, n_blocks=2)
