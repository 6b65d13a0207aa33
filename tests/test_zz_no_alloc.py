"""The allocation-free smoothing entry point (qattn_smooth_quant_noalloc,
whose partial sums live in the library's static device array) against
qattn_smooth_quant with a caller workspace, through the C ABI: every output
bit for bit, on two calls in a row, the second on a smaller problem (the
array keeps the first call's contents)."""

import numpy as np
import pytest
import torch

import bit_quantized_attention_amd as qa
from synthetic import make_case

pytestmark = pytest.mark.gpu

OUTS = ["q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "q_pool", "k_pool"]


def _outputs(p, dev):
    nqb, nkb = p.N // 128, p.N // 64
    return {
        "q_i8": torch.empty((p.B, p.Hq, p.N, p.d), dtype=torch.int8, device=dev),
        "q_scale": torch.empty((p.B, p.Hq, nqb), dtype=torch.float32, device=dev),
        "k_i8": torch.empty((p.B, p.Hkv, p.N, p.d), dtype=torch.int8, device=dev),
        "k_scale": torch.empty((p.B, p.Hkv, nkb), dtype=torch.float32, device=dev),
        "k_mean": torch.empty((p.B, p.Hkv, p.d), dtype=torch.float32, device=dev),
        "q_pool": torch.empty((p.B, p.Hq, nqb, p.d), dtype=torch.float32, device=dev),
        "k_pool": torch.empty((p.B, p.Hkv, nkb, p.d), dtype=torch.float32, device=dev),
    }


def _both(p, t):
    dev = torch.device("cuda:0")
    q, k = t["q"].to(dev), t["k"].to(dev)
    prob = qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal)
    ref, got = _outputs(p, dev), _outputs(p, dev)
    ws = torch.empty(qa.qattn_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    qa.qattn_smooth_quant(prob, q, k, *(ref[n] for n in OUTS), ws)
    # outputs poisoned first, so that a skipped write shows
    for x in got.values():
        x.fill_(-7)
    qa.qattn_smooth_quant_noalloc(prob, q, k, *(got[n] for n in OUTS))
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(ref[n], got[n]), n
    return got


def test_noalloc_matches_the_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qa.load()
    # first a long problem (8 MiB of partial sums in the static array), then a
    # smaller one of another head size and dtype, whose partial sums overwrite
    # only the start of the array
    p1, t1 = make_case(B=1, Hq=16, Hkv=8, N=65536, d=128, dtype="bf16", causal=True, seed=91,
                       k_offset_std=3.0, outliers=4)
    got1 = _both(p1, t1)
    p2, t2 = make_case(B=2, Hq=4, Hkv=2, N=640, d=64, dtype="f16", causal=False, seed=92,
                       k_offset_std=2.0)
    got2 = _both(p2, t2)
    assert got2["k_mean"].shape == (2, 2, 64)
    # the channel means are exact: one more check against the host sum of K
    km = t2["k"].double().mean(dim=2).float().numpy()
    assert np.array_equal(got2["k_mean"].cpu().numpy(), km)
    assert got1["k_mean"].shape == (1, 8, 128)
