/*
 * qattn -- 8-bit quantized, optionally block-sparse attention forward (prefill)
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are explainer pages; each entry point below cites the
 * passage that defines its operation):
 *   1. smooth K by subtracting its per-channel mean over tokens, and quantize
 *      Q (128-token blocks) and smoothed K (64-token blocks) to INT8 with one
 *      fp32 scale per block;
 *   2. optionally score every (query block, key block) pair by the dot product
 *      of their INT8-quantized mean vectors and keep, per query block, the
 *      first block, the diagonal blocks and the top fraction of the rest;
 *   3. compute S = Q K^T on INT8 matrix cores, an online base-2 softmax, and
 *      P V on FP16/BF16 matrix cores with FP32 accumulation, visiting only the
 *      kept key blocks when a mask is given -- or, promoting instead of
 *      skipping, computing the kept blocks' Q K^T on 16-bit matrix cores and
 *      every other block through the INT8 path.
 *
 * Conventions shared by every entry point:
 *   - Layouts are contiguous row-major: Q and O are [B, Hq, N, d]; K and V are
 *     [B, Hkv, N, d]. Query head hq reads kv head hq / (Hq / Hkv).
 *   - Causal masking is top-left aligned: key j is visible to query i iff
 *     j <= i.
 *   - Every tensor pointer is a device pointer owned by the caller and must be
 *     16-byte aligned. The library allocates and frees nothing and keeps no
 *     mutable state; calls on different streams may run concurrently.
 *   - `stream` is a hipStream_t passed as void* (NULL: the default stream).
 *     Work is enqueued on it; no call synchronizes.
 *   - Arguments are validated on the host before any HIP call. A failing
 *     validation returns its status and enqueues nothing. A launch failure
 *     returns QATTN_ERR_DEVICE. No C++ exception crosses this interface.
 *   - Supported: d in {64, 128}; N a positive multiple of 128; dtype f16 or
 *     bf16 for Q, K, V and O.
 */
#ifndef QATTN_H
#define QATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QATTN_OK = 0,
  QATTN_ERR_NULL = 1,        /* a required pointer is NULL                  */
  QATTN_ERR_SHAPE = 2,       /* a dimension <= 0, or Hq % Hkv != 0          */
  QATTN_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned     */
  QATTN_ERR_UNSUPPORTED = 4, /* d not 64/128, N % 128 != 0, unknown dtype   */
  QATTN_ERR_ARG = 5,         /* bad flag, keep ratio, max_keep or workspace */
  QATTN_ERR_DEVICE = 6,      /* a HIP launch reported an error              */
  QATTN_ERR_SCRATCH = 7      /* beyond the allocation-free entry point's static scratch */
} qattn_status_t;

typedef enum { QATTN_F16 = 0, QATTN_BF16 = 1 } qattn_dtype_t;

typedef struct {
  int32_t B;      /* batch                                  */
  int32_t Hq;     /* query heads                            */
  int32_t Hkv;    /* key/value heads, divides Hq            */
  int32_t N;      /* tokens (queries = keys)                */
  int32_t d;      /* head dimension                         */
  int32_t dtype;  /* qattn_dtype_t of Q, K, V and O         */
  int32_t causal; /* 0 or 1                                 */
} qattn_problem_t;

/* Quantization block lengths (tokens) and the key tile of the online softmax. */
#define QATTN_Q_BLOCK 128
#define QATTN_K_BLOCK 64
#define QATTN_KV_TILE 64
/* Online-softmax reference threshold (log2 units): a row's exponent reference
 * moves to the running max only when the max exceeds it by more than this. */
#define QATTN_SOFTMAX_REF_THRESHOLD 8

/* Message for a status code (static storage, never NULL). */
const char* qattn_status_str(qattn_status_t status);

/* Library version string. */
const char* qattn_version(void);

/* Device workspace bytes that qattn_smooth_quant (per-chunk exact partial
 * sums of K) and qattn_block_mask (INT8 codes and scales of the pooled
 * vectors) need for `p`; one buffer of this size serves both calls when they
 * run in stream order. 0 when `p` is NULL or invalid. */
size_t qattn_workspace_bytes(const qattn_problem_t* p);

/* Length of each kept list that qattn_block_mask writes for a keep ratio of
 * keep_num / keep_den: min(N/64, 3 + ceil((N/64) * keep_num / keep_den)).
 * Returns -1 for an invalid problem or ratio. */
int32_t qattn_max_keep(const qattn_problem_t* p, int32_t keep_num, int32_t keep_den);

/*
 * qattn_smooth_quant -- K smoothing and per-block INT8 quantization.
 *
 * Defined by the SageAttention explainer (aibr.jp/archives/102657), sections 2
 * and 3: K is smoothed so that extreme per-channel values do not inflate the
 * quantization scale, and the attention inputs are quantized to 8 bits. The
 * pages give no formulas; this library computes:
 *   k_mean[b,hk,c] = fl32(fl64(fl64(exact sum over t of K[b,hk,t,c]) / N))
 *   Ks             = fl32(fl32(K) - k_mean)            (per channel)
 *   per block X (Q: 128 tokens x d of one (b, hq); Ks: 64 tokens x d):
 *     scale = fl32(amax|X| / 127), or 1.0 when that is 0;
 *     code  = clamp(round-half-even(x / scale), -127, 127), x / scale exact.
 *   optional pooled block means (inputs of qattn_block_mask):
 *     q_pool[b,hq,i,c] = fl32(fl64(exact sum over the 128 tokens of Q) / 128)
 *     k_pool[b,hk,j,c] = fl32(fl64(fl64(exact sum over the 64 tokens of K) / 64)
 *                             - k_mean[b,hk,c])
 *   The sums are exact (hence independent of reduction order) whenever, per
 *   channel, max|K| / (smallest nonzero |K|) < 2^64 -- always for f16.
 *
 * In:  q [B,Hq,N,d], k [B,Hkv,N,d] in p->dtype.
 * Out: q_i8 [B,Hq,N,d] int8, q_scale [B,Hq,N/128] f32,
 *      k_i8 [B,Hkv,N,d] int8, k_scale [B,Hkv,N/64] f32, k_mean [B,Hkv,d] f32,
 *      q_pool [B,Hq,N/128,d] f32 and k_pool [B,Hkv,N/64,d] f32 (each may be
 *      NULL: not computed).
 * workspace: device scratch of at least qattn_workspace_bytes(p) bytes,
 *      overwritten; it must not be shared with a concurrent call.
 * Errors: NULL for a missing required pointer; SHAPE/UNSUPPORTED for the
 *      problem; ALIGN; ARG when workspace_bytes is too small or causal is not
 *      0/1; DEVICE on launch failure.
 */
qattn_status_t qattn_smooth_quant(const qattn_problem_t* p, const void* q, const void* k,
                                  int8_t* q_i8, float* q_scale, int8_t* k_i8,
                                  float* k_scale, float* k_mean, float* q_pool,
                                  float* k_pool, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * qattn_smooth_quant_noalloc -- qattn_smooth_quant without a workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * kernels and results as qattn_smooth_quant (bit for bit); the exact
 * partial K sums live in a static device array of QATTN_NOALLOC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends (its address
 * is looked up on the device's first call). No hipMalloc, hipFree or other
 * allocation happens in this call.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and corrupt each other's k_mean. Every
 * partial sum is written before it is read, so nothing needs clearing between
 * calls.
 * Arguments, layouts and outputs as qattn_smooth_quant.
 * Errors: NULL; SHAPE/UNSUPPORTED; ALIGN; SCRATCH when the partial sums,
 *      B * Hkv * ceil(N/128) * d * 16 bytes, exceed the array (for example
 *      B = 1, Hkv = 8, d = 128 fits up to N = 131072); DEVICE.
 */
#define QATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
qattn_status_t qattn_smooth_quant_noalloc(const qattn_problem_t* p, const void* q, const void* k,
                                          int8_t* q_i8, float* q_scale, int8_t* k_i8,
                                          float* k_scale, float* k_mean, float* q_pool,
                                          float* k_pool, void* stream);

/*
 * qattn_block_mask -- per query block, the key blocks to keep.
 *
 * Score: the ThriftAttention summary (gist.science/ja/paper/2605.23081),
 * technical summary, method (heuristic block selection): a (query block i,
 * key block j) pair is scored by the dot product of the blocks' mean vectors
 * and the top-k pairs are selected. Skipping the rest while keeping the first
 * (sink) and diagonal (local) blocks: the SALE explainer
 * (aibr.jp/archives/118208), section 3. This library computes, per
 * (b, hq, i) with hk = hq / (Hq/Hkv):
 *   each pooled vector is INT8-quantized on its own (the rule above, over its
 *   d channels); dot = exact integer dot product of the codes;
 *   score[i,j] = fl32(fl32(float(dot) * q_scale_i) * k_scale_j);
 *   valid = { j : 64 j <= 128 i + 127 } if causal, else all j < N/64;
 *   forced = valid & { 0, 2i, 2i+1 };
 *   kcount = ceil(|valid| * keep_num / keep_den) (integer arithmetic);
 *   kept = forced + the top min(kcount, |valid \ forced|) of valid \ forced by
 *          (score descending, j ascending).
 * In:  q_pool [B,Hq,N/128,d], k_pool [B,Hkv,N/64,d] f32 (from qattn_smooth_quant).
 * Out: kv_idx [B,Hq,N/128,max_keep] int32, kept blocks ascending then -1;
 *      kv_cnt [B,Hq,N/128] int32, number of kept blocks.
 * workspace: device scratch of at least qattn_workspace_bytes(p) bytes,
 *      overwritten; it must not be shared with a concurrent call.
 * Errors: NULL; SHAPE; UNSUPPORTED also when N > 131072; ALIGN; ARG when
 *      keep_num < 0, keep_den <= 0, keep_num > keep_den,
 *      max_keep < qattn_max_keep(p, keep_num, keep_den), or the workspace is
 *      too small; DEVICE.
 */
qattn_status_t qattn_block_mask(const qattn_problem_t* p, const float* q_pool,
                                const float* k_pool, int32_t keep_num, int32_t keep_den,
                                int32_t max_keep, int32_t* kv_idx, int32_t* kv_cnt,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * qattn_fwd -- quantized attention forward.
 *
 * Kernel: the SageAttention explainer (aibr.jp/archives/102657), section 3
 * (INT8 matrix products for Q K^T, 16-bit products for P V, on the matrix
 * units) and section 4 (FlashAttention-style tiling); online softmax merge as
 * in the ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
 * summary, method. This library computes, per (b, hq), per query block of 128
 * rows and per key tile of 64 keys in ascending order (all causally visible
 * tiles when dense; the kept tiles when kv_idx is given):
 *   S = q_codes k_codes^T (exact int32);
 *   alpha = fl32(fl32(q_scale * fl32(log2(e)/sqrt(d))) * k_scale);
 *   s = S * alpha, -inf where the key is masked;
 *   c = max(m, rowmax s); m' = c if c > m + QATTN_SOFTMAX_REF_THRESHOLD
 *   (or m = -inf), else m' = m; P = exp2(s - m'), P_hat = P rounded to V's
 *   dtype; l = l * exp2(m - m') + rowsum P (before the rounding);
 *   acc = acc * exp2(m - m') + P_hat V (fp32);
 *   O = acc / l rounded to V's dtype; lse = ln2 * (m + log2 l), the natural
 *   log-sum-exp of the smoothed, dequantized logits (S * alpha / log2(e)).
 * In:  q_i8, q_scale, k_i8, k_scale as written by qattn_smooth_quant;
 *      v [B,Hkv,N,d] in p->dtype; kv_idx/kv_cnt from qattn_block_mask or NULL
 *      for dense (both NULL, or both non-NULL with the max_keep they were
 *      written with). Kept-list entries outside [0, N/64), entries past the
 *      query block's causal range, and counts above max_keep are ignored.
 * Out: o [B,Hq,N,d] in p->dtype; lse [B,Hq,N] f32 or NULL. A query row with
 *      no visible key gets O = 0 and lse = -inf.
 *      A block listed more than once is attended as often as it is listed
 *      (its weight counts that many times in O and lse, as in the oracle).
 * Errors: NULL; SHAPE/UNSUPPORTED, also UNSUPPORTED with a mask when
 *      N > 131072 (N/64 > 2048 blocks); ALIGN; ARG when exactly one of
 *      kv_idx/kv_cnt is NULL, or with a mask when max_keep < 1 or
 *      max_keep > 2048; DEVICE.
 */
qattn_status_t qattn_fwd(const qattn_problem_t* p, const int8_t* q_i8, const float* q_scale,
                         const int8_t* k_i8, const float* k_scale, const void* v,
                         const int32_t* kv_idx, const int32_t* kv_cnt, int32_t max_keep,
                         void* o, float* lse, void* stream);

/*
 * qattn_fwd_promoted -- promote instead of skip: the kept blocks at 16-bit
 * Q K^T, every other visible block through the INT8 path of qattn_fwd.
 *
 * The ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
 * summary, method: the top-k block pairs are computed in 16-bit precision,
 * the remaining pairs at low precision, and both are merged by a
 * FlashAttention-2 style online softmax; its implementation paragraph runs
 * the low-precision blocks first and the promoted ones after. Here the low
 * path is INT8 and the kept list (typically from qattn_block_mask) names the
 * promoted blocks. Per (b, hq) and query block i of 128 rows:
 *   promoted = the distinct kept-list entries (the first kv_cnt of them) that
 *              are in [0, N/64) and causally visible; low = every other
 *              visible 64-key block;
 *   first the low blocks, ascending, exactly as qattn_fwd's dense path;
 *   then each promoted block, ascending, as two 32-key halves, with
 *     S16 = q . k over the caller's 16-bit Q and K rows (fp32 accumulation),
 *     cq  = fl32(fl32(log2(e)/sqrt(d)) * (q . k_mean)) (fp32 accumulation),
 *     s   = fl32(log2(e)/sqrt(d)) * S16 - cq,
 *   which is the smoothed logit q . (k - k_mean) in the INT8 path's units,
 *   taken through the same online-softmax step as an INT8 tile;
 *   O and lse as in qattn_fwd.
 * In:  q_i8, q_scale, k_i8, k_scale, k_mean as written by qattn_smooth_quant
 *      for these q and k; q [B,Hq,N,d] and k [B,Hkv,N,d] in p->dtype (the
 *      inputs of that call); v [B,Hkv,N,d]; kv_idx [B,Hq,N/128,max_keep] and
 *      kv_cnt [B,Hq,N/128] int32 (entries outside the range or the causal
 *      range, duplicates and counts above max_keep are ignored).
 * Out: o [B,Hq,N,d] in p->dtype; lse [B,Hq,N] f32 or NULL.
 * Errors: NULL for any missing pointer but lse; SHAPE/UNSUPPORTED, also
 *      UNSUPPORTED when N > 131072; ALIGN; ARG when max_keep < 1 or
 *      max_keep > 2048; DEVICE.
 */
qattn_status_t qattn_fwd_promoted(const qattn_problem_t* p, const int8_t* q_i8,
                                  const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                  const void* q, const void* k, const float* k_mean,
                                  const void* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int32_t max_keep, void* o, float* lse, void* stream);

/*
 * qattn_fwd_promoted_fp4 -- promote instead of skip with an MX FP4 low path:
 * the kept blocks at 16-bit Q K^T, every other visible block at 4-bit Q K^T.
 *
 * The ThriftAttention summary (gist.science/ja/paper/2605.23081), technical
 * summary, method: the top-k block pairs at 16-bit precision, the remaining
 * pairs in a 4-bit format (NVFP4 on the page's hardware), one online-softmax
 * merge, the low blocks first. Here the 4-bit format is OCP MX FP4 (the
 * format of qattn_block_mask_lowbit: E2M1 codes, one E8M0 exponent per 32
 * channels) of the raw Q and the smoothed K, on CDNA4's FP4 matrix cores.
 * Per (b, hq) and query block of 128 rows, the plan and order are those of
 * qattn_fwd_promoted; a low 64-key tile's logit is
 *   s = fl32(log2(e)/sqrt(d)) * S4, S4 the dot product of the dequantized
 *   4-bit query and key vectors (exact in fp32 while the exponents of the
 *   summed 32-channel groups span less than about ten binades),
 * formed with one fma into the exponent; P is rounded to V's dtype and P V
 * runs at 16 bits as on the INT8 path. The call first writes the MX FP4 codes
 * of q and of k - k_mean into the workspace, then runs the forward.
 * In:  q [B,Hq,N,d], k [B,Hkv,N,d], v [B,Hkv,N,d] in p->dtype; k_mean
 *      [B,Hkv,d] f32 from qattn_smooth_quant; kv_idx [B,Hq,N/128,max_keep],
 *      kv_cnt [B,Hq,N/128] int32 as for qattn_fwd_promoted.
 * Out: o [B,Hq,N,d] in p->dtype; lse [B,Hq,N] f32 or NULL.
 * workspace: device scratch for the codes, overwritten (the layout of the
 *      low-bit mask's workspace without its block scores:
 *      qattn_lowbit_workspace_bytes(p) - 4*B*Hq*(N/128)*(N/64) bytes suffice,
 *      qattn_lowbit_workspace_bytes(p) always does); not to be shared with a
 *      concurrent call.
 * Errors: NULL for any missing pointer but lse; SHAPE/UNSUPPORTED, also
 *      UNSUPPORTED when N > 131072; ALIGN; ARG when max_keep < 1,
 *      max_keep > 2048 or the workspace is too small; DEVICE.
 */
qattn_status_t qattn_fwd_promoted_fp4(const qattn_problem_t* p, const void* q, const void* k,
                                      const float* k_mean, const void* v, const int32_t* kv_idx,
                                      const int32_t* kv_cnt, int32_t max_keep, void* o, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * qattn_block_mask_lowbit -- per query block, the key blocks to keep, scored
 * from element-level 4-bit estimates.
 *
 * The SALE explainer (aibr.jp/archives/118208), sections 2 and 3: every
 * query-key product is estimated with 4-bit quantized Q and K, the estimates
 * are turned into a block-sparse plan, and the sink and local patterns are
 * kept (qattn_block_mask_patterns adds the predicted vertical and slash lines
 * to such a plan). This library computes, per (b, hq):
 *   the raw Q and the smoothed K, Ks = fl32(K) - k_mean, in OCP MX FP4: per 32
 *   consecutive channels a shared exponent E = floor(log2 amax) - 2 (at least
 *   -127; -127 for an all-zero group) and E2M1 elements, x / 2^E rounded to
 *   nearest-even on {0, .5, 1, 1.5, 2, 3, 4, 6} and saturated at 6;
 *   est(q, k) = the dot product of the dequantized vectors (the matrix cores
 *   accumulate it in fp32);
 *   score[i, j] = max of est over the causally visible pairs of query block i
 *   (128 rows) and key block j (64 keys);
 *   kept = the rule of qattn_block_mask (first and diagonal blocks forced,
 *   then the top ceil(|valid| * keep_num / keep_den) of the rest by score,
 *   ties to the lower block index).
 * In:  q [B,Hq,N,d], k [B,Hkv,N,d] in p->dtype; k_mean [B,Hkv,d] f32 from
 *      qattn_smooth_quant.
 * Out: kv_idx [B,Hq,N/128,max_keep] int32 (kept blocks ascending, then -1),
 *      kv_cnt [B,Hq,N/128] int32; scores [B,Hq,N/128,N/64] f32 or NULL (only
 *      the causally valid entries are written).
 * workspace: at least qattn_lowbit_workspace_bytes(p) bytes of device memory,
 *      overwritten; not to be shared with a concurrent call.
 * Errors: NULL (scores may be NULL); SHAPE/UNSUPPORTED, also UNSUPPORTED when
 *      N > 131072; ALIGN; ARG for the keep ratio, max_keep below
 *      qattn_max_keep(p, keep_num, keep_den), or a small workspace; DEVICE.
 */
size_t qattn_lowbit_workspace_bytes(const qattn_problem_t* p);

qattn_status_t qattn_block_mask_lowbit(const qattn_problem_t* p, const void* q, const void* k,
                                       const float* k_mean, int32_t keep_num, int32_t keep_den,
                                       int32_t max_keep, int32_t* kv_idx, int32_t* kv_cnt,
                                       float* scores, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * qattn_block_mask_patterns -- add the predicted vertical and slash lines of
 * each head to every query block's kept list.
 *
 * The SALE explainer (aibr.jp/archives/118208), sections 1 and 3: the method
 * also predicts vertical lines (key positions every query needs) and slash
 * lines (a fixed query-key distance) from the attention map's tendencies.
 * Here the tendencies are the votes of the per-query-block selections. Per
 * (b, hq), with i a query block (128 rows) and j a key block (64 keys):
 *   kept(i) = the entries among the first min(kv_cnt, max_keep) of list i
 *     that are valid key blocks for i (0 <= j < N/64; j <= 2i + 1 when
 *     causal), once each;
 *   forced(i) = {0, 2i, 2i + 1} (the blocks every plan of qattn_block_mask
 *     holds by rule, which carry no information);
 *   each j in kept(i) \ forced(i) gives one vote to key block j (vertical)
 *     and one to offset o = 2i - j (slash; negative past the diagonal);
 *   the lines are the n_vertical key blocks and the n_slash offsets with the
 *     most votes, at least two each, ties to the lower block or offset;
 *   out(i) = kept(i), the valid vertical blocks and the valid blocks 2i - o
 *     of the slash offsets, ascending.
 * In:  kv_idx [B,Hq,N/128,max_keep], kv_cnt [B,Hq,N/128] int32 (e.g. from
 *      qattn_block_mask or qattn_block_mask_lowbit).
 * Out: kv_idx_out [B,Hq,N/128,max_keep_out] (ascending, then -1),
 *      kv_cnt_out [B,Hq,N/128]; lines [B,Hq,n_vertical + n_slash] int32: the
 *      vertical blocks in rank order (-1 where fewer qualify), then the slash
 *      offsets in rank order (INT32_MIN where fewer qualify). The outputs must
 *      not overlap the inputs. lines may be NULL when no line is asked for.
 * Errors: NULL; SHAPE/UNSUPPORTED, also UNSUPPORTED when N > 131072; ALIGN;
 *      ARG when n_vertical or n_slash is outside [0, QATTN_MAX_PATTERN_LINES],
 *      max_keep < 1, max_keep_out < min(N/64, max_keep + n_vertical +
 *      n_slash), or an output overlaps an input; DEVICE.
 */
#define QATTN_MAX_PATTERN_LINES 64

qattn_status_t qattn_block_mask_patterns(const qattn_problem_t* p, const int32_t* kv_idx,
                                         const int32_t* kv_cnt, int32_t max_keep,
                                         int32_t n_vertical, int32_t n_slash, int32_t* kv_idx_out,
                                         int32_t* kv_cnt_out, int32_t max_keep_out,
                                         int32_t* lines, void* stream);

/*
 * qattn_stripe_select -- per query block, the key positions within a
 * threshold of the anchor (AnchorAttention-style stripes).
 *
 * The AnchorAttention explainer (aibr.jp/archives/118418), section 3: an
 * approximate maximum score (the anchor) from the initial tokens and a local
 * window; every other position is kept when its score comes within a
 * threshold of the anchor, by direct comparison without a sort, selecting
 * discrete key positions. This library computes, per (b, hq, query block i):
 *   score(k) = fl32(fl32(dot * sq) * sk[k/64]): dot the exact product of the
 *     INT8 codes of the block's mean query (q_pool, quantized on its own as in
 *     qattn_block_mask) and of key k (k_i8), sk = k_scale;
 *   region = the first 64 keys and keys 128 i .. 128 i + 127, causally valid;
 *   anchor = max of score over the region;
 *   kept = region + { k causally valid : score(k) >= fl32(anchor - theta) },
 *     ascending; when that exceeds max_keys, the region and the lowest-index
 *     other keys.
 * In:  q_pool [B,Hq,N/128,d] f32, k_i8 [B,Hkv,N,d], k_scale [B,Hkv,N/64] from
 *      qattn_smooth_quant; theta (score units, may be +inf).
 * Out: key_idx [B,Hq,N/128,max_keys] int32 (ascending, then -1),
 *      key_cnt [B,Hq,N/128] int32.
 * Errors: NULL; SHAPE/UNSUPPORTED, also UNSUPPORTED when N > 65536; ALIGN;
 *      ARG when theta is NaN or max_keys is outside [192, 3072]; DEVICE.
 */
qattn_status_t qattn_stripe_select(const qattn_problem_t* p, const float* q_pool,
                                   const int8_t* k_i8, const float* k_scale, float theta,
                                   int32_t max_keys, int32_t* key_idx, int32_t* key_cnt,
                                   void* stream);

/*
 * qattn_fwd_stripes -- quantized attention over gathered (discrete) keys.
 *
 * The AnchorAttention explainer (aibr.jp/archives/118418), section 3: the
 * attention reads the selected discrete key and value positions instead of
 * contiguous blocks. This library computes qattn_fwd's online softmax per
 * query block over its key list taken 64 entries at a time (the last group
 * may be shorter), in list order, with each key's own block scale:
 *   s = fl32(S * fl32(fl32(q_scale * fl32(log2(e)/sqrt(d))) * k_scale[k/64])),
 *   -inf where the key is past the row (causal).
 * In:  q_i8, q_scale, k_i8, k_scale from qattn_smooth_quant; v; key_idx /
 *      key_cnt (e.g. from qattn_stripe_select; entries outside [0, N) or past
 *      the query block's causal range and counts above max_keys are ignored;
 *      a repeated entry is attended as often as it appears; lists should be
 *      ascending: the first whole 64-entry groups holding no key past the
 *      block's first row skip the causal test).
 * Out: o [B,Hq,N,d] in p->dtype; lse [B,Hq,N] f32 or NULL.
 * Errors: NULL; SHAPE/UNSUPPORTED, also UNSUPPORTED when N > 65536; ALIGN;
 *      ARG when max_keys is outside [1, 3072]; DEVICE.
 */
qattn_status_t qattn_fwd_stripes(const qattn_problem_t* p, const int8_t* q_i8,
                                 const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                 const void* v, const int32_t* key_idx, const int32_t* key_cnt,
                                 int32_t max_keys, void* o, float* lse, void* stream);

/*
 * qattn_head_error -- per-head error proxy of the INT8 Q K^T (adaptive
 * per-head precision, data-free).
 *
 * The SageAttention explainer (aibr.jp/archives/102657), sections 1-4, names
 * adaptive quantization, set per layer or head so that the parts that need it
 * keep more precision, as the method's third ingredient; it gives no rule.
 * This library measures, per (b, hq), over a fixed sample of up to 64 query
 * rows (row 128*floor(u*nqb/nsq) + (37u+11) mod 128, u < nsq = min(nqb, 64))
 * and up to 256 keys (key 64*floor(w*nkb/nsk) + (29w+5) mod 64,
 * w < nsk = min(nkb, 256)), all pairs, visible or not:
 *   s8  = fl32(S * alpha): S the exact INT8 code product, alpha as in
 *         qattn_fwd (the INT8 path's base-2 logit);
 *   s16 = c * (q . k - q . k_mean), c = fl32(log2(e)/sqrt(d)), on the 16-bit
 *         Q and K with fp32 accumulation (the 16-bit path's logit);
 *   head_err = sqrt(mean (s8 - s16)^2) (fp32, fixed summation order);
 *   head_hi  = head_err > threshold ? 1 : 0.
 * In:  q_i8, q_scale, k_i8, k_scale, k_mean from qattn_smooth_quant of q, k
 *      (the 16-bit inputs, p->dtype).
 * Out: head_err [B,Hq] f32; head_hi [B,Hq] int32 or NULL.
 * Errors: NULL (head_hi may be NULL); SHAPE/UNSUPPORTED; ALIGN; ARG when the
 *      threshold is negative or not finite; DEVICE.
 */
qattn_status_t qattn_head_error(const qattn_problem_t* p, const int8_t* q_i8,
                                const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                const void* q, const void* k, const float* k_mean,
                                float threshold, float* head_err, int32_t* head_hi,
                                void* stream);

/*
 * qattn_fwd_adaptive -- attention with the precision of Q K^T chosen per
 * head: every visible block of a head with head_hi[b,hq] != 0 at 16-bit
 * Q K^T, every block of the other heads through the INT8 path.
 *
 * Same computation as qattn_fwd_promoted with a kept list holding all visible
 * blocks for the flagged heads and none for the others (same source
 * passages, plus the SageAttention explainer's adaptive quantization, sections
 * 1-4). A flagged head's tiles run as 32-key halves in ascending order; an
 * unflagged head's as 64-key INT8 tiles in ascending order.
 * In:  as qattn_fwd_promoted; head_hi [B,Hq] int32 (e.g. from
 *      qattn_head_error).
 * Out: o [B,Hq,N,d] in p->dtype; lse [B,Hq,N] f32 or NULL.
 * Errors: NULL for any missing pointer but lse; SHAPE/UNSUPPORTED, also
 *      UNSUPPORTED when N > 131072; ALIGN; DEVICE.
 */
qattn_status_t qattn_fwd_adaptive(const qattn_problem_t* p, const int8_t* q_i8,
                                  const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                  const void* q, const void* k, const float* k_mean,
                                  const void* v, const int32_t* head_hi, void* o, float* lse,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QATTN_H */
