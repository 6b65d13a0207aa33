"""GPU parity of adaptive per-head precision (qattn_head_error and
qattn_fwd_adaptive) against the oracle, through the C ABI.

The per-head error is compared with the oracle's fp64 value (relative 1e-4);
the flags (error > threshold) are compared except at near-ties. Each side then
runs its own flags: the oracle the promoted emulation with all-or-nothing
lists, the GPU qattn_fwd_adaptive; the outputs are compared on the heads whose
flags agree, at the bars of the other paths.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import make_case
from parity_util import (TOL_EMU, COS_MIN, KERNEL_TAU, log, out_err, cos, to_np, emulate_both,
                         check_out)

pytestmark = pytest.mark.gpu

THRESHOLD = 0.019  # splits the heads of the Llama-shaped law (errors 0.016-0.022)

CASES = [
    ("bf16-d128-causal-gqa4-N1024", dict(B=1, Hq=8, Hkv=2, N=1024, d=128, dtype="bf16",
                                         causal=True, seed=61, k_offset_std=3.0, outliers=4)),
    ("f16-d64-nc-B2-N640", dict(B=2, Hq=4, Hkv=4, N=640, d=64, dtype="f16", causal=False,
                                seed=62, k_offset_std=2.0)),
    ("bf16-d64-causal-mqa-N256", dict(B=1, Hq=4, Hkv=1, N=256, d=64, dtype="bf16", causal=True,
                                      seed=63, k_offset_std=3.0, outliers=2)),
    ("bf16-d128-causal-N16384", dict(B=1, Hq=2, Hkv=1, N=16384, d=128, dtype="bf16",
                                     causal=True, seed=64, k_offset_std=3.0, outliers=4)),
]


def _gpu(qa, p, t):
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev, with_lse=True)
    plan.smooth_quant(q, k)
    err = torch.empty((p.B, p.Hq), dtype=torch.float32, device=dev)
    hi = torch.empty((p.B, p.Hq), dtype=torch.int32, device=dev)
    return dev, q, k, v, plan, err, hi


def _oracle_err(p, t):
    sq = oracle.smooth_quant(t["q"], t["k"])
    e = oracle.head_error(sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"], t["q"], t["k"],
                          sq["k_mean"], p.Hq, p.Hkv)
    return sq, e


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_head_error_matches_oracle(gpu_lib, name, kw):
    p, t = make_case(**kw)
    log(f"head error {name}")
    qa = gpu_lib
    dev, q, k, v, plan, err, hi = _gpu(qa, p, t)
    qa.qattn_head_error(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                        plan.k_mean, THRESHOLD, err, hi)
    torch.cuda.synchronize()
    _, e = _oracle_err(p, t)
    g = to_np(err).astype(np.float64)
    rel = float(np.abs(g - e).max() / e.max())
    log(f"  err range {e.min():.4f}-{e.max():.4f}, max rel diff {rel:.2e}")
    assert rel < 1e-4
    near = np.abs(e - THRESHOLD) <= 1e-4 * THRESHOLD
    assert np.array_equal(to_np(hi)[~near] != 0, (e > THRESHOLD)[~near])


def test_head_error_scales_exactly_with_q(gpu_lib):
    p, t = make_case(B=1, Hq=4, Hkv=2, N=512, d=128, dtype="bf16", causal=True, seed=65,
                     k_offset_std=3.0, outliers=4)
    qa = gpu_lib
    out = []
    for scale in (1, 4):
        t2 = dict(t, q=t["q"] * scale)  # exact in bf16
        dev, q, k, v, plan, err, hi = _gpu(qa, p, t2)
        qa.qattn_head_error(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                            plan.k_mean, 0.0, err, None)
        torch.cuda.synchronize()
        out.append(err.clone())
    assert torch.equal(out[1], 4 * out[0])


@pytest.mark.parametrize("name,kw", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_fwd_adaptive_matches_emulation(gpu_lib, name, kw):
    p, t = make_case(**kw)
    log(f"adaptive fwd {name}")
    qa = gpu_lib
    dev, q, k, v, plan, err, hi = _gpu(qa, p, t)
    qa.qattn_head_error(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                        plan.k_mean, THRESHOLD, err, hi)
    o = torch.empty_like(q)
    qa.qattn_fwd_adaptive(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, hi, o, plan.lse)
    torch.cuda.synchronize()
    sq, e = _oracle_err(p, t)
    flags = e > THRESHOLD
    agree = (to_np(hi) != 0) == flags
    idx, cnt = oracle.adaptive_lists(flags, p.N, p.causal)
    (_, O_pre, lse_emu), (_, O_pre0, _) = emulate_both(
        oracle.emulate_promoted_attention, sq["q_i8"], sq["q_scale"], sq["k_i8"], sq["k_scale"],
        t["q"], t["k"], sq["k_mean"], t["v"], p.causal, p.Hq, p.Hkv, idx, cnt)
    O_ex, _ = oracle.exact_attention(t["q"], t["k"], t["v"], p.causal)
    og = to_np(o)
    check_out(og[agree], O_pre[agree], O_pre0[agree], p.dtype, v=t["v"])
    c = cos(og[agree], O_ex[agree])
    dl = float(np.abs(to_np(plan.lse)[agree] - lse_emu[agree]).max())
    log(f"  flagged {int(flags.sum())}/{flags.size} heads, lse_err={dl:.2e} cos_exact={c:.6f}")
    assert dl < 1e-4 and c >= COS_MIN


def test_fwd_adaptive_extremes_are_the_other_paths(gpu_lib):
    # no head flagged = the dense INT8 kernel; every head flagged = the
    # promoted path with every block kept; bit for bit
    p, t = make_case(B=1, Hq=4, Hkv=2, N=1024, d=128, dtype="bf16", causal=True, seed=66,
                     k_offset_std=3.0)
    log("adaptive fwd with no / all heads flagged")
    qa = gpu_lib
    dev, q, k, v, plan, err, hi = _gpu(qa, p, t)
    o_dense = torch.empty_like(q)
    qa.qattn_fwd(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, v, None, None, 0,
                 o_dense, None)
    o_none, o_all, o_prom = (torch.empty_like(q) for _ in range(3))
    zeros = torch.zeros((1, 4), dtype=torch.int32, device=dev)
    ones = torch.ones((1, 4), dtype=torch.int32, device=dev)
    qa.qattn_fwd_adaptive(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, zeros, o_none, None)
    qa.qattn_fwd_adaptive(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, ones, o_all, None)
    nqb, nkb = p.N // 128, p.N // 64
    idx = torch.arange(nkb, dtype=torch.int32, device=dev).repeat(1, 4, nqb, 1).contiguous()
    cnt = torch.full((1, 4, nqb), nkb, dtype=torch.int32, device=dev)
    qa.qattn_fwd_promoted(plan.p, plan.q_i8, plan.q_scale, plan.k_i8, plan.k_scale, q, k,
                          plan.k_mean, v, idx, cnt, nkb, o_prom, None)
    torch.cuda.synchronize()
    assert torch.equal(o_none, o_dense)
    assert torch.equal(o_all, o_prom)
