"""Exact attention and the step-by-step quantized path (oracle; test infrastructure only).

``exact_attention`` is the plain definition the method approximates:
O = softmax(Q K^T / sqrt(d)) V per (batch, query head), in fp64, with query
head hq reading kv head hq // (Hq / Hkv), an optional causal mask (key j is
visible to query i iff j <= i) and an optional block mask (a key is visible
only when its 64-key block is in the query's 128-query block keep list).

``emulate_attention`` follows the quantized kernel of the SageAttention
explainer (aibr.jp/archives/102657, sections 2-3: INT8 product for Q K^T, a
16-bit product for P V, FlashAttention-style tiling per section 4) with the
online softmax merge of the ThriftAttention summary (gist.science/ja/paper/
2605.23081, technical summary, method: merged as in FlashAttention-2). Readings
where the pages are silent:

* per query block of 128 rows and per key tile of ``kv_tile`` keys, ascending:
  S = q_codes . k_codes^T (exact integers);
* dequantization folds the softmax temperature and the change to base 2:
  c = fl32(log2(e) / sqrt(d)), alpha_q = fl32(q_scale * c),
  alpha = fl32(alpha_q * k_scale[key block]), s = fl32(S * alpha);
  masked scores are -inf;
* the exponent reference m of each row: m_cand = max(m, rowmax(s)); the
  reference moves to m_cand only when m_cand > fl32(m + tau) (always on the
  first visible key, m = -inf); otherwise it stays, so P may exceed 1 by up to
  2^tau. tau = 0 is the textbook per-tile update; the kernel uses tau = 8
  (its rescale of the accumulator is then almost never needed). In exact
  arithmetic the result does not depend on the reference;
* P = fl32(exp2(fl32(s - m_new))); P_hat = P rounded to nearest-even in V's
  dtype (the 16-bit operand of the P V product);
  corr = fl32(exp2(fl32(m_old - m_new))) (1 when the reference did not move);
  l = l * corr + sum(P), the row sum of P before its 16-bit rounding, as in
  FlashAttention-2's online softmax; acc = acc * corr + P_hat V, accumulated
  in fp64 (the kernel accumulates in fp32: the 16-bit products are exact in
  either). With V = 1 the output is sum(P_hat) / sum(P), within the unit
  roundoff of V's dtype of 1;
* O = round_dtype(fl32(acc / l)); lse = ln(2) * (m + log2(l)), the natural log
  normalizer of the smoothed, dequantized logits.
"""

from __future__ import annotations

import math

import numpy as np

from .quant import Q_BLOCK, K_BLOCK, _as_f64
from .rounding import round_to_dtype

LOG2E = 1.4426950408889634


def softmax_scale_log2(d: int) -> np.float32:
    """fl32(log2(e) / sqrt(d)): the scale folded into the INT8 dequantization."""
    return np.float32(LOG2E / math.sqrt(d))


def _kept_keys_mask(kv_idx_row, cnt, N):
    keep = np.zeros(N, dtype=bool)
    for j in kv_idx_row[:cnt]:
        keep[int(j) * K_BLOCK:(int(j) + 1) * K_BLOCK] = True
    return keep


def exact_attention(q, k, v, causal: bool, kv_idx=None, kv_cnt=None, blocks=None):
    """fp64 softmax attention. Returns (O fp64 [B,Hq,N,d], lse fp64 [B,Hq,N]).

    ``blocks`` optionally restricts the work to a list of (b, hq, i) query
    blocks; other entries are NaN.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, N, d = q64.shape
    Hkv = k64.shape[1]
    group = Hq // Hkv
    O = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    nqb = N // Q_BLOCK
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nqb)]
    inv_sqrt_d = 1.0 / math.sqrt(d)
    keys = np.arange(N)
    for b, hq, i in blocks:
        hk = hq // group
        r0, r1 = i * Q_BLOCK, (i + 1) * Q_BLOCK
        s = (q64[b, hq, r0:r1] @ k64[b, hk].T) * inv_sqrt_d
        vis = np.ones((Q_BLOCK, N), dtype=bool)
        if causal:
            vis &= keys[None, :] <= np.arange(r0, r1)[:, None]
        if kv_idx is not None:
            vis &= _kept_keys_mask(kv_idx[b, hq, i], kv_cnt[b, hq, i], N)[None, :]
        s = np.where(vis, s, -np.inf)
        mx = np.max(s, axis=1, keepdims=True)
        mx_safe = np.where(np.isfinite(mx), mx, 0.0)
        p = np.exp(s - mx_safe)
        den = p.sum(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            O[b, hq, r0:r1] = np.where(den > 0, (p @ v64[b, hk]) / den, 0.0)
            lse[b, hq, r0:r1] = np.where(den[:, 0] > 0, mx_safe[:, 0] + np.log(den[:, 0]), -np.inf)
    return O, lse


def _kv_tiles_dense(i: int, N: int, causal: bool, kv_tile: int):
    n_tiles = N // kv_tile
    if not causal:
        return list(range(n_tiles))
    last_key = Q_BLOCK * i + Q_BLOCK - 1
    return list(range(min(n_tiles, last_key // kv_tile + 1)))


def _dtypes(v, p_dtype, out_dtype):
    """P's and O's rounding dtypes, defaulting to V's 16-bit dtype."""
    vdt = None
    try:
        import torch
        if isinstance(v, torch.Tensor):
            vdt = {torch.bfloat16: "bf16", torch.float16: "f16"}.get(v.dtype)
    except ImportError:  # pragma: no cover
        pass
    p_dtype = p_dtype or vdt
    out_dtype = out_dtype or vdt
    if p_dtype is None or out_dtype is None:
        raise ValueError("p_dtype/out_dtype needed when V is not a 16-bit torch tensor")
    return p_dtype, out_dtype


def _online_step(m, l, acc, s, vt, p_dtype, tau):
    """One step of the online softmax over a tile of fp32 base-2 logits.

    m [rows] f32 reference, l [rows] f64 row sums, acc [rows, d] f64;
    s [rows, keys] f32 logits (-inf where masked); vt [keys, d] f64 values.
    The reference rule, P, P_hat, corr, l and acc as in the module docstring.
    """
    ninf = np.float32(-np.inf)
    m_cand = np.maximum(m, s.max(axis=1))
    move = m_cand > (m + np.float32(tau)).astype(np.float32)
    m_new = np.where(move, m_cand, m).astype(np.float32)
    live = np.isfinite(m_new)
    arg = np.where(live[:, None], (s - np.where(live, m_new, 0)[:, None]).astype(np.float32), ninf)
    P = np.exp2(arg.astype(np.float64)).astype(np.float32)
    P_hat = round_to_dtype(P, p_dtype).astype(np.float64)
    dm = np.where(np.isfinite(m), (m - np.where(live, m_new, 0)).astype(np.float32), ninf)
    corr = np.where(np.isfinite(m), np.exp2(dm.astype(np.float64)).astype(np.float32), 0.0)
    corr = np.where(live, corr, 1.0).astype(np.float64)
    l = l * corr + P.astype(np.float64).sum(axis=1)
    acc = acc * corr[:, None] + P_hat @ vt
    return m_new, l, acc


def _finish(m, l, acc):
    """O before its final rounding (f32) and lse (f64) from the final state."""
    with np.errstate(invalid="ignore", divide="ignore"):
        o32 = np.where(l[:, None] > 0, acc / l[:, None], 0.0).astype(np.float32)
        lse = np.where(l > 0, math.log(2.0) * (m.astype(np.float64) + np.log2(l)), -np.inf)
    return o32, lse


def emulate_attention(q_i8, q_scale, k_i8, k_scale, v, causal: bool, Hq: int, Hkv: int,
                      kv_idx=None, kv_cnt=None, kv_tile: int = K_BLOCK,
                      p_dtype: str | None = None, out_dtype: str | None = None,
                      blocks=None, tau: float = 0.0):
    """The quantized path, step by step.

    q_i8 [B,Hq,N,d] int8, q_scale [B,Hq,N/128] f32, k_i8 [B,Hkv,N,d] int8,
    k_scale [B,Hkv,N/64] f32, v [B,Hkv,N,d] in the 16-bit dtype (torch tensor
    or fp64 array). ``kv_idx``/``kv_cnt`` select the sparse path (the kept
    64-key blocks, ascending); then ``kv_tile`` must be 64.
    ``p_dtype`` is the dtype P is rounded to ("bf16", "f16", or "f32" for no
    16-bit rounding); ``out_dtype`` the output's. Both default to V's dtype,
    which must then be given as a torch tensor. ``tau`` is the reference
    threshold of the online softmax (log2 units, see the module docstring).

    Returns (O rounded [B,Hq,N,d] f32 values, O before the final rounding
    [B,Hq,N,d] f32, lse [B,Hq,N] f64). ``blocks`` restricts the work to a list
    of (b, hq, i); other entries are NaN.
    """
    p_dtype, out_dtype = _dtypes(v, p_dtype, out_dtype)
    v64 = _as_f64(v)
    B, _, N, d = q_i8.shape
    group = Hq // Hkv
    sparse = kv_idx is not None
    if sparse and kv_tile != K_BLOCK:
        raise ValueError("the sparse path iterates 64-key blocks")
    if N % kv_tile or kv_tile % K_BLOCK:
        raise ValueError("kv_tile must be a multiple of 64 dividing N")
    c = softmax_scale_log2(d)
    nqb = N // Q_BLOCK
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
        qc = q_i8[b, hq, r0:r0 + Q_BLOCK].astype(np.float64)
        alpha_q = np.float32(np.float32(q_scale[b, hq, i]) * c)
        m = np.full(Q_BLOCK, ninf, dtype=np.float32)
        l = np.zeros(Q_BLOCK)
        acc = np.zeros((Q_BLOCK, d))
        if sparse:
            tiles = [int(j) for j in kv_idx[b, hq, i, :kv_cnt[b, hq, i]]]
        else:
            tiles = _kv_tiles_dense(i, N, causal, kv_tile)
        for t in tiles:
            k0 = t * kv_tile
            keys = np.arange(k0, k0 + kv_tile)
            # INT8 Q K^T: exact integers (|S| <= d * 127^2 < 2^53)
            S = qc @ k_i8[b, hk, k0:k0 + kv_tile].astype(np.float64).T
            kb = keys // K_BLOCK
            alpha = (alpha_q * np.asarray(k_scale[b, hk, kb], dtype=np.float32)).astype(np.float32)
            s = (S.astype(np.float32) * alpha[None, :]).astype(np.float32)
            if causal:
                s = np.where(keys[None, :] <= rows[:, None], s, ninf)
            m, l, acc = _online_step(m, l, acc, s, v64[b, hk, k0:k0 + kv_tile], p_dtype, tau)
        o32, lse[b, hq, r0:r0 + Q_BLOCK] = _finish(m, l, acc)
        O_pre[b, hq, r0:r0 + Q_BLOCK] = o32
        O[b, hq, r0:r0 + Q_BLOCK] = round_to_dtype(o32, out_dtype)
    return O, O_pre, lse


def promote_plan(kv_idx_row, cnt: int, i: int, N: int, causal: bool):
    """The two tile lists of query block i on the promoted path.

    promoted: the distinct entries of the kept list (its first ``cnt``) that
    name a 64-key block in range and causally visible to the block, ascending;
    low: every other visible block, ascending. Together they cover each
    visible block exactly once.
    """
    visible = _kv_tiles_dense(i, N, causal, K_BLOCK)
    vis = set(visible)
    promoted = sorted({int(j) for j in kv_idx_row[:cnt] if int(j) in vis})
    low = [t for t in visible if t not in set(promoted)]
    return low, promoted


def emulate_promoted_attention(q_i8, q_scale, k_i8, k_scale, q, k, k_mean, v, causal: bool,
                               Hq: int, Hkv: int, kv_idx, kv_cnt,
                               p_dtype: str | None = None, out_dtype: str | None = None,
                               blocks=None, tau: float = 0.0):
    """Promote instead of skip: the kept blocks at 16-bit Q K^T, the rest INT8.

    The ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
    summary, method: the top-k block pairs are computed in 16-bit precision,
    every other pair at low precision, and the two are merged by the online
    softmax; its implementation paragraph runs the low-precision blocks first
    and the promoted ones after. Here the low path is the INT8 path of
    ``emulate_attention`` and the kept list comes from the block mask.
    Readings where the page is silent:

    * per query block, the low blocks (``promote_plan``) are visited first,
      ascending, as 64-key tiles exactly as in ``emulate_attention``;
    * then each promoted block, ascending, as two 32-key halves in order;
      a half's logits use the original 16-bit q and k and the K mean:
      s = fl32(c * (q . k - q . k_mean)) with c = fl32(log2(e)/sqrt(d)) and
      the products and sums exact (fp64 here; the kernel accumulates in
      fp32). Subtracting q . k_mean puts these logits in the same frame as the
      smoothed INT8 logits (q . (k - k_mean)); without it the two paths would
      disagree by a per-row constant;
    * the online-softmax step of each tile or half, the epilogue and lse are
      those of ``emulate_attention``.

    q [B,Hq,N,d], k [B,Hkv,N,d] (16-bit torch tensors or fp64 arrays),
    k_mean [B,Hkv,d] f32 (the smoothing mean); kv_idx [B,Hq,N/128,max_keep],
    kv_cnt [B,Hq,N/128]. Returns (O, O_pre, lse) as ``emulate_attention``.
    """
    p_dtype, out_dtype = _dtypes(v, p_dtype, out_dtype)
    v64, q64, k64 = _as_f64(v), _as_f64(q), _as_f64(k)
    mean64 = np.asarray(k_mean, dtype=np.float32).astype(np.float64)
    B, _, N, d = q_i8.shape
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
        qc = q_i8[b, hq, r0:r0 + Q_BLOCK].astype(np.float64)
        alpha_q = np.float32(np.float32(q_scale[b, hq, i]) * c)
        m = np.full(Q_BLOCK, ninf, dtype=np.float32)
        l = np.zeros(Q_BLOCK)
        acc = np.zeros((Q_BLOCK, d))
        low, promoted = promote_plan(kv_idx[b, hq, i], int(kv_cnt[b, hq, i]), i, N, causal)
        for t in low:
            k0 = t * K_BLOCK
            keys = np.arange(k0, k0 + K_BLOCK)
            S = qc @ k_i8[b, hk, k0:k0 + K_BLOCK].astype(np.float64).T
            alpha = np.float32(alpha_q * np.float32(k_scale[b, hk, t]))
            s = (S.astype(np.float32) * alpha).astype(np.float32)
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


def head_error_sample(N: int):
    """The (query row, key) sample of ``head_error``.

    Up to 64 query rows, one from each of as many evenly spaced query blocks
    (block i_u = floor(u * nqb / nsq), row 128*i_u + (37*u + 11) mod 128), and
    up to 256 keys, one from each of as many evenly spaced key blocks (block
    j_w = floor(w * nkb / nsk), key 64*j_w + (29*w + 5) mod 64). Every
    (row, key) combination is a sampled pair, causally visible or not: the
    statistic is about the quantization of the logits, not the mask.
    """
    nqb, nkb = N // Q_BLOCK, N // K_BLOCK
    nsq, nsk = min(nqb, 64), min(nkb, 256)
    rows = np.array([Q_BLOCK * ((u * nqb) // nsq) + (37 * u + 11) % Q_BLOCK for u in range(nsq)])
    keys = np.array([K_BLOCK * ((w * nkb) // nsk) + (29 * w + 5) % K_BLOCK for w in range(nsk)])
    return rows, keys


def head_error(q_i8, q_scale, k_i8, k_scale, q, k, k_mean, Hq: int, Hkv: int):
    """Data-free per-head error proxy of the INT8 Q K^T (adaptive precision).

    The SageAttention explainer (aibr.jp/archives/102657), sections 1-4, names
    adaptive quantization as its third ingredient: the quantization is set per
    layer or head so that the heads that need it keep more precision, and the
    adaptive version is faster at no loss. The page gives no rule. Here the
    rule uses only the head's own Q and K: over the pairs of
    ``head_error_sample``,
      s8  = fl32(S * alpha), S the exact INT8 code product and alpha as in
            ``emulate_attention`` (the INT8 path's base-2 logit);
      s16 = c * (q . k - q . k_mean), c = fl32(log2(e)/sqrt(d)) (the 16-bit
            path's logit, exact here);
      err = sqrt(mean over the pairs of (s8 - s16)^2), in log2 units,
    i.e. the RMS logit error the INT8 path adds in that head (a P is off by a
    factor 2^(s8 - s16)). Returns err [B, Hq] fp64.
    """
    q64, k64 = _as_f64(q), _as_f64(k)
    mean64 = np.asarray(k_mean, dtype=np.float32).astype(np.float64)
    B, _, N, d = q_i8.shape
    group = Hq // Hkv
    c = softmax_scale_log2(d)
    rows, keys = head_error_sample(N)
    err = np.zeros((B, Hq))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // group
            S = q_i8[b, hq, rows].astype(np.float64) @ k_i8[b, hk, keys].astype(np.float64).T
            alpha_q = (np.asarray(q_scale[b, hq, rows // Q_BLOCK], dtype=np.float32) * c
                       ).astype(np.float32)
            alpha = (alpha_q[:, None] * np.asarray(k_scale[b, hk, keys // K_BLOCK],
                                                   dtype=np.float32)[None, :]).astype(np.float32)
            s8 = (S.astype(np.float32) * alpha).astype(np.float64)
            qr = q64[b, hq, rows]
            s16 = float(c) * (qr @ k64[b, hk, keys].T - (qr @ mean64[b, hk])[:, None])
            err[b, hq] = math.sqrt(np.mean((s8 - s16) ** 2))
    return err


def adaptive_lists(head_hi, N: int, causal: bool):
    """Kept lists that promote every visible block of the flagged heads and
    none of the others (head_hi [B, Hq] bool): the adaptive forward is the
    promoted forward with these lists."""
    B, Hq = head_hi.shape
    nqb, nkb = N // Q_BLOCK, N // K_BLOCK
    idx = np.full((B, Hq, nqb, nkb), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            if not head_hi[b, h]:
                continue
            for i in range(nqb):
                vis = _kv_tiles_dense(i, N, causal, K_BLOCK)
                idx[b, h, i, :len(vis)] = vis
                cnt[b, h, i] = len(vis)
    return idx, cnt
