"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same inputs (optionally on a slice of heads / query blocks), and
the comparison metrics with their tolerances."""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import bit_quantized_attention_amd as qa
import oracle

# Output tolerance of the quantized path against its emulation (max-abs-relative
# of the difference before the final 16-bit rounding, see out_err below) and the
# cosine-similarity floor against exact fp64 attention.
TOL_EMU = 2e-3
COS_MIN = 0.999
# The online-softmax reference rule of the kernel (a lazy rescale: a row's
# exponent reference moves only when the running max passes it by more than
# 8 in log2 units), written here as the literal of that documented reading and
# not read from the library. The textbook FlashAttention-2 update moves the
# reference at every new maximum (tau = 0). Every forward comparison is made
# against both emulations and both must meet TOL_EMU.
KERNEL_TAU = 8.0
TEXTBOOK_TAU = 0.0


def log(msg: str):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def ulp16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit dtype at |x| (bf16: 8 significant bits, f16: 11)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    bits = 8 if dtype == "bf16" else 11
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14 if dtype == "f16" else 2.0 ** -126)))
    return np.exp2(e - (bits - 1))


def out_err(o_gpu: np.ndarray, o_emu_pre: np.ndarray, dtype: str) -> float:
    """max_i max(0, |o_gpu - o_emu_pre| - ulp/2) / max|o_emu_pre|.

    o_gpu is the kernel's 16-bit output, o_emu_pre the emulation's output before
    its own final rounding. Removing half an output ulp removes exactly the part
    of the difference that the final rounding alone can make; what remains is
    bounded by the difference before rounding."""
    d = np.abs(o_gpu.astype(np.float64) - o_emu_pre.astype(np.float64))
    d = np.maximum(0.0, d - 0.5 * ulp16(o_emu_pre, dtype))
    return float(d.max() / np.abs(o_emu_pre).max())


def emulate_both(fn, *args, **kw):
    """fn(*args, tau=KERNEL_TAU, **kw) and fn(*args, tau=TEXTBOOK_TAU, **kw)."""
    return fn(*args, tau=KERNEL_TAU, **kw), fn(*args, tau=TEXTBOOK_TAU, **kw)


def p_roundoff(dtype: str) -> float:
    """Unit roundoff of P's 16-bit type (P is rounded to V's dtype)."""
    return 2.0 ** -9 if dtype == "bf16" else 2.0 ** -12


def textbook_bound(o_ref: np.ndarray, vmax: float, dtype: str) -> float:
    """Bound on out_err between two online softmaxes that differ only in their
    exponent reference (the lazy rule and the textbook update), relative to
    max|o_ref|: each output is sum(P_hat v) / sum(P) with P_hat = P (1 + e),
    |e| <= u, so each lies within u * max|v| of the unrounded-P result, and the
    two within 2 u max|v| of each other; TOL_EMU on top covers the kernel's own
    distance to its emulation."""
    return TOL_EMU + 2.0 * p_roundoff(dtype) * vmax / float(np.abs(o_ref).max())


def check_out(o_gpu: np.ndarray, pre_kernel: np.ndarray, pre_textbook: np.ndarray, dtype: str,
              what: str = "", v=None) -> float:
    """out_err against the emulation of the kernel's online-softmax rule
    (asserted within TOL_EMU) and against the textbook online softmax (logged,
    and asserted within TOL_EMU or, when V is given, within textbook_bound:
    the two emulations themselves differ by up to about 2.3e-3 where O is small
    against V, e.g. long non-causal rows). Returns the first."""
    e8 = out_err(o_gpu, pre_kernel, dtype)
    e0 = out_err(o_gpu, pre_textbook, dtype)
    vmax = None if v is None else float(np.abs(to_np(v) if isinstance(v, torch.Tensor) else v).max())
    bound = TOL_EMU if vmax is None else max(TOL_EMU, textbook_bound(pre_textbook, vmax, dtype))
    log(f"  {what}err_vs_emu(tau=8)={e8:.3e} err_vs_textbook(tau=0)={e0:.3e} "
        f"(textbook bound {bound:.2e})")
    assert e8 <= TOL_EMU, f"{what}out_err {e8:.3e} against the emulation (tau=8)"
    assert e0 <= bound, f"{what}out_err {e0:.3e} against the textbook online softmax (tau=0)"
    return e8


def max_abs_rel(a: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(a.astype(np.float64) - ref.astype(np.float64)).max() / np.abs(ref).max())


def cos(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy()


def run_gpu(qa, p, t, sparse=None, pools=None, with_lse=True, promote=False, low4=False):
    """The whole path on cuda:0 through the C ABI; returns (plan, o) on device."""
    dev = torch.device("cuda:0")
    q, k, v = (t[x].to(dev) for x in "qkv")
    plan = qa.Plan(qa.problem(p.B, p.Hq, p.Hkv, p.N, p.d, p.dtype, p.causal), dev,
                   sparse=sparse, with_lse=with_lse, pools=pools, promote=promote, low4=low4)
    o = torch.empty_like(q)
    plan.run(q, k, v, o)
    torch.cuda.synchronize()
    return plan, o


def head_slice(t, p, b: int, hqs):
    """Inputs restricted to batch b, query heads hqs (all of one kv head) and that kv head."""
    hk = hqs[0] // p.group
    assert all(h // p.group == hk for h in hqs)
    sub = {"q": t["q"][b:b + 1, list(hqs)].contiguous(),
           "k": t["k"][b:b + 1, hk:hk + 1].contiguous(),
           "v": t["v"][b:b + 1, hk:hk + 1].contiguous()}
    return sub, hk


def same_lists(gi, gc, idx, cnt, ties):
    """Per (b, hq, i): do the GPU's kept list (gi, gc) and the oracle's (idx,
    cnt) agree? Asserts that they do wherever the oracle reports no near-tie,
    and that the counts always agree; returns the agreement mask, so that the
    attention outputs are compared only where both sides used the same list."""
    assert np.array_equal(gc, cnt)
    agree = np.all(gi == idx, axis=-1)
    assert np.all(agree | ties)
    return agree


def block_rows(mask_bh_i: np.ndarray) -> np.ndarray:
    """[B, Hq, nqb] block mask -> [B, Hq, N] row mask (128 rows per block)."""
    return np.repeat(mask_bh_i, 128, axis=-1)
