"""Promote instead of skip with an MX FP4 low path (oracle; test
infrastructure only).

The ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
summary, method: the top-k block pairs are computed in 16-bit precision, the
remaining pairs in a 4-bit format (NVFP4 on the page's hardware), and both are
merged by the FlashAttention-2 style online softmax; its implementation
paragraph runs the low-precision blocks first and the promoted ones after.
``attention.emulate_promoted_attention`` takes INT8 as the low path; this one
takes 4 bits. Readings where the page is silent:

* the 4-bit format is OCP MX FP4, the one CDNA4's matrix cores take: the Q
  and smoothed-K codes of ``lowbit.lowbit_inputs`` (E2M1 elements with one
  E8M0 exponent per 32 channels; the raw Q and fl32(K) - k_mean);
* a low tile's logit is s = fl32(c * fl32(S4)), S4 the exact dot product of
  the dequantized 4-bit query and key vectors and c = fl32(log2(e)/sqrt(d)):
  the smoothed keys put it in the same frame as the promoted logits
  q . (k - k_mean), as for the INT8 low path;
* only Q K^T changes precision; P is rounded to V's 16-bit type and P V runs
  at 16 bits as on the INT8 path (the page's two-level quantization of P for
  a 4-bit P V product is not taken);
* the plan, the order (low 64-key tiles ascending, then each promoted block as
  two 32-key halves), the online-softmax step, the epilogue and lse are those
  of ``emulate_promoted_attention``.
"""

from __future__ import annotations

import numpy as np

from .quant import Q_BLOCK, K_BLOCK, _as_f64
from .rounding import round_to_dtype
from .attention import (softmax_scale_log2, promote_plan, _online_step, _finish, _dtypes)
from .lowbit import lowbit_inputs


def emulate_promoted_fp4_attention(q, k, k_mean, v, causal: bool, Hq: int, Hkv: int, kv_idx,
                                   kv_cnt, p_dtype: str | None = None,
                                   out_dtype: str | None = None, blocks=None, tau: float = 0.0):
    """The kept blocks at 16-bit Q K^T, every other visible block at MX FP4.

    q [B,Hq,N,d], k [B,Hkv,N,d] (16-bit torch tensors or fp64 arrays), k_mean
    [B,Hkv,d] f32 (the smoothing mean), v [B,Hkv,N,d]; kv_idx
    [B,Hq,N/128,max_keep], kv_cnt [B,Hq,N/128]. Returns (O, O_pre, lse) as
    ``emulate_attention``.
    """
    p_dtype, out_dtype = _dtypes(v, p_dtype, out_dtype)
    v64, q64, k64 = _as_f64(v), _as_f64(q), _as_f64(k)
    mean64 = np.asarray(k_mean, dtype=np.float32).astype(np.float64)
    q4, k4 = lowbit_inputs(q, k, k_mean)      # dequantized MX FP4, fp64
    B, _, N, d = q64.shape
    group = Hq // Hkv
    c = softmax_scale_log2(d)
    c64 = float(c)
    nqb = N // Q_BLOCK
    half = K_BLOCK // 2
    O = np.full((B, Hq, N, d), np.nan, dtype=np.float32)
    O_pre = np.full((B, Hq, N, d), np.nan, dtype=np.float32)
    lse = np.full((B, Hq, N), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nqb)]
    ninf = np.float32(-np.inf)
    for b, hq, i in blocks:
        hk = hq // group
        r0 = i * Q_BLOCK
        rows = np.arange(r0, r0 + Q_BLOCK)
        m = np.full(Q_BLOCK, ninf, dtype=np.float32)
        l = np.zeros(Q_BLOCK)
        acc = np.zeros((Q_BLOCK, d))
        low, promoted = promote_plan(kv_idx[b, hq, i], int(kv_cnt[b, hq, i]), i, N, causal)
        q4rows = q4[b, hq, r0:r0 + Q_BLOCK]
        for t in low:
            k0 = t * K_BLOCK
            keys = np.arange(k0, k0 + K_BLOCK)
            S4 = (q4rows @ k4[b, hk, k0:k0 + K_BLOCK].T).astype(np.float32)  # exact, then fl32
            s = (c * S4).astype(np.float32)
            if causal:
                s = np.where(keys[None, :] <= rows[:, None], s, ninf)
            m, l, acc = _online_step(m, l, acc, s, v64[b, hk, k0:k0 + K_BLOCK], p_dtype, tau)
        qrows = q64[b, hq, r0:r0 + Q_BLOCK]
        qm = qrows @ mean64[b, hk]                  # q . k_mean per row
        for t in promoted:
            for hf in range(2):
                k0 = t * K_BLOCK + hf * half
                keys = np.arange(k0, k0 + half)
                raw = qrows @ k64[b, hk, k0:k0 + half].T
                s = (c64 * (raw - qm[:, None])).astype(np.float32)
                if causal:
                    s = np.where(keys[None, :] <= rows[:, None], s, ninf)
                m, l, acc = _online_step(m, l, acc, s, v64[b, hk, k0:k0 + half], p_dtype, tau)
        o32, lse[b, hq, r0:r0 + Q_BLOCK] = _finish(m, l, acc)
        O_pre[b, hq, r0:r0 + Q_BLOCK] = o32
        O[b, hq, r0:r0 + Q_BLOCK] = round_to_dtype(o32, out_dtype)
    return O, O_pre, lse
