"""K smoothing and per-block INT8 quantization (oracle; test infrastructure only).

Follows the SageAttention explainer (aibr.jp/archives/102657), sections 2 and 3:
K is smoothed before quantization so that large per-channel values do not blow
up the quantization scale, and the attention inputs Q and K are quantized to 8
bits. The pages give neither the smoothing formula nor the quantizer; the
readings used here are:

* smoothing: subtract from every token of K its per-channel mean over all N
  tokens of that (batch, kv head). Because q.m is the same for every key of a
  query row, softmax is unchanged by the subtraction (shift invariance).
* mean: the exact sum over tokens, rounded to fp64, divided by N in fp64, then
  rounded to fp32:  m = fl32(fl64(fl64(sum_t K[t, c]) / N)).
* smoothed K: Ks = fl32(fl32(K) - m).
* quantizer, per block (Q: 128 tokens x d of one (batch, head); K: 64 tokens x
  d): amax = max |x| over the block, scale = fl32(amax / 127); when that is 0
  (an all-zero block, or an amax so small that the quotient underflows) the
  scale is 1.0. code = clamp(round-half-even(x / scale), -127, 127), where
  x / scale is the exact real quotient (symmetric signed INT8, no zero point).
* pooled block vectors for the block mask:
  q_pool[i, c] = fl32(fl64(fl64(sum over the 128 tokens of Q[t, c]) / 128)),
  k_pool[j, c] = fl32(fl64(fl64(fl64(sum over the 64 tokens of K[t, c]) / 64) - m[c]))
  i.e. the block mean of the smoothed K, taken in fp64 and rounded once.
"""

from __future__ import annotations

import numpy as np

from .rounding import exact_sum, exact_sums_rows

Q_BLOCK = 128
K_BLOCK = 64


def _as_f64(x) -> np.ndarray:
    """Upcast a torch tensor or array of the 16-bit input dtype to fp64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def k_channel_mean(k) -> np.ndarray:
    """Per-(batch, kv head, channel) mean of K over tokens -> fp32 [B, Hkv, d]."""
    k64 = _as_f64(k)
    B, H, N, d = k64.shape
    cols = np.ascontiguousarray(np.moveaxis(k64, 2, 3)).reshape(B * H * d, N)
    sums = exact_sums_rows(cols)
    mean64 = sums / np.float64(N)
    return mean64.astype(np.float32).reshape(B, H, d)


def quantize_block(x32: np.ndarray):
    """Quantize one block of float32 values to INT8 codes with one fp32 scale."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    scale = np.float32(amax / np.float32(127.0))
    if scale == 0:
        scale = np.float32(1.0)
    # fp64 holds the exact quotient of two float32 values closely enough that
    # rounding it to an integer gives the same code as rounding the exact
    # quotient (the quotient is either exactly a half-integer, which fp64
    # represents, or at least 2^-26 away from one, far beyond fp64 rounding).
    quot = x32.astype(np.float64) / np.float64(scale)
    codes = np.clip(np.rint(quot), -127, 127).astype(np.int8)
    return codes, scale


def _quantize_blocks(x32: np.ndarray, block: int):
    """Apply ``quantize_block`` to every ``block``-token block of [B,H,N,d]."""
    B, H, N, d = x32.shape
    nb = N // block
    codes = np.empty((B, H, N, d), dtype=np.int8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                c, s = quantize_block(x32[b, h, j * block:(j + 1) * block])
                codes[b, h, j * block:(j + 1) * block] = c
                scales[b, h, j] = s
    return codes, scales


def _block_col_sums(x64: np.ndarray, block: int) -> np.ndarray:
    """Exact-then-fp64-rounded sums over tokens of every block and channel."""
    B, H, N, d = x64.shape
    nb = N // block
    blk = x64.reshape(B, H, nb, block, d)
    cols = np.ascontiguousarray(np.moveaxis(blk, 3, 4)).reshape(B * H * nb * d, block)
    return exact_sums_rows(cols).reshape(B, H, nb, d)


def q_block_pool(q) -> np.ndarray:
    """Mean of Q over each 128-token block, per channel -> fp32 [B, Hq, N/128, d]."""
    q64 = _as_f64(q)
    sums = _block_col_sums(q64, Q_BLOCK)
    return (sums / np.float64(Q_BLOCK)).astype(np.float32)


def k_block_pool(k, k_mean: np.ndarray) -> np.ndarray:
    """Mean of the smoothed K over each 64-token block -> fp32 [B, Hkv, N/64, d]."""
    k64 = _as_f64(k)
    sums = _block_col_sums(k64, K_BLOCK)
    mean_blk = sums / np.float64(K_BLOCK)
    return (mean_blk - k_mean.astype(np.float64)[:, :, None, :]).astype(np.float32)


def smooth_quant(q, k, pools: bool = False):
    """The whole pre-processing stage.

    Returns a dict with q_i8 [B,Hq,N,d] int8, q_scale [B,Hq,N/128] f32,
    k_i8 [B,Hkv,N,d] int8, k_scale [B,Hkv,N/64] f32, k_mean [B,Hkv,d] f32 and,
    when ``pools``, q_pool [B,Hq,N/128,d] f32 and k_pool [B,Hkv,N/64,d] f32.
    """
    q64 = _as_f64(q)
    k64 = _as_f64(k)
    m = k_channel_mean(k64)
    ks32 = k64.astype(np.float32) - m[:, :, None, :]          # fp32 subtraction
    q32 = q64.astype(np.float32)                              # exact upcast
    q_i8, q_scale = _quantize_blocks(q32, Q_BLOCK)
    k_i8, k_scale = _quantize_blocks(ks32, K_BLOCK)
    out = dict(q_i8=q_i8, q_scale=q_scale, k_i8=k_i8, k_scale=k_scale, k_mean=m)
    if pools:
        out["q_pool"] = q_block_pool(q64)
        out["k_pool"] = k_block_pool(k64, m)
    return out


def pool_vector_quant(p: np.ndarray):
    """INT8-quantize each pooled vector (last axis, d channels) on its own.

    Same rule as ``quantize_block`` with the vector as the block. Returns
    (codes int8 [..., d], scales f32 [...]).
    """
    p = np.asarray(p, dtype=np.float32)
    lead = p.shape[:-1]
    flat = p.reshape(-1, p.shape[-1])
    codes = np.empty(flat.shape, dtype=np.int8)
    scales = np.empty(flat.shape[0], dtype=np.float32)
    for r in range(flat.shape[0]):
        codes[r], scales[r] = quantize_block(flat[r])
    return codes.reshape(p.shape), scales.reshape(lead)


__all__ = ["k_channel_mean", "quantize_block", "smooth_quant", "pool_vector_quant",
           "q_block_pool", "k_block_pool", "exact_sum", "Q_BLOCK", "K_BLOCK"]
