// Internal declarations shared by the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qattn {

constexpr int kQBlock = 128;     // query tokens per quantization block
constexpr int kKBlock = 64;      // key tokens per quantization block
constexpr int kKsumChunk = 128;  // tokens per partial K sum

struct Shape {
  int B, Hq, Hkv, N, d;
  int bf16;    // 1: bfloat16, 0: float16
  int causal;  // 0/1
  int nqb() const { return N / kQBlock; }
  int nkb() const { return N / kKBlock; }
  int nchunk() const { return (N + kKsumChunk - 1) / kKsumChunk; }
};

// Bytes of exact partial sums that launch_smooth_quant needs.
inline size_t ksum_workspace_bytes(const Shape& s) {
  return (size_t)s.B * s.Hkv * s.nchunk() * s.d * 2 * sizeof(double);
}

hipError_t launch_smooth_quant(const Shape& s, const void* q, const void* k, int8_t* q_i8,
                               float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                               float* q_pool, float* k_pool, void* workspace,
                               hipStream_t stream);

// Size of the static device scratch of the allocation-free smoothing entry
// point (one array per GPU, held until the process ends).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;

// launch_smooth_quant with its partial sums in that static scratch of the
// current device (its address looked up once per device, never allocated).
hipError_t launch_smooth_quant_noalloc(const Shape& s, const void* q, const void* k, int8_t* q_i8,
                                       float* q_scale, int8_t* k_i8, float* k_scale,
                                       float* k_mean, float* q_pool, float* k_pool,
                                       hipStream_t stream);

// Bytes of pooled-vector INT8 codes and scales that launch_block_mask needs.
size_t mask_workspace_bytes(const Shape& s);
// Largest N/64 the block mask supports.
int mask_max_nkb();

hipError_t launch_block_mask(const Shape& s, const float* q_pool, const float* k_pool,
                             int keep_num, int keep_den, int max_keep, int32_t* kv_idx,
                             int32_t* kv_cnt, void* workspace, hipStream_t stream);

// Kept lists from precomputed block scores [B*Hq*nqb][nkb] (the pooled
// mask's selection rule).
hipError_t launch_select_scores(const Shape& s, const float* scores, int keep_num, int keep_den,
                                int max_keep, int32_t* kv_idx, int32_t* kv_cnt,
                                hipStream_t stream);

// Workspace of the element-level 4-bit estimator (MX FP4 Q and K codes and
// exponents, plus the block scores unless the caller takes them).
size_t lowbit_workspace_bytes(const Shape& s, bool with_scores);

// The element-level 4-bit block scores and the kept lists chosen from them;
// scores (optional) receives the block scores.
hipError_t launch_lowbit_mask(const Shape& s, const void* q, const void* k, const float* k_mean,
                              int keep_num, int keep_den, int max_keep, int32_t* kv_idx,
                              int32_t* kv_cnt, float* scores, void* workspace,
                              hipStream_t stream);

// Longest kept list qattn_fwd accepts (entries per query block); also the
// most 64-key blocks (N / 64) the promoted path supports.
int fwd_max_sparse_tiles();

// MX FP4 codes and exponents of Q and the smoothed K (the low-bit workspace
// layout): q4 [B*Hq*N][d/2], qe [B*Hq*N][d/32], k4 [B*Hkv*N][d/2],
// ke [B*Hkv*N][d/32].
struct Fp4Codes {
  const uint8_t* q4;
  const uint8_t* qe;
  const uint8_t* k4;
  const uint8_t* ke;
};

// Dense (kv_idx NULL), sparse (kv_idx set, q16 NULL), promoted (kv_idx, q16,
// k16 and k_mean set; low4 set: the low tiles at MX FP4 instead of INT8),
// adaptive (head_hi, q16, k16 and k_mean set, kv_idx NULL) or gathered-key
// (gather, kv_idx / kv_cnt / max_keep the key lists) attention forward.
hipError_t launch_attn_fwd(const Shape& s, const int8_t* q_i8, const float* q_scale,
                           const int8_t* k_i8, const float* k_scale, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, int max_keep,
                           const void* q16, const void* k16, const float* k_mean,
                           const int32_t* head_hi, bool gather, void* o, float* lse,
                           hipStream_t stream, const Fp4Codes* low4 = nullptr);

// MX FP4 quantization of the raw Q and the smoothed K into the low-bit
// workspace, and the codes' addresses there.
hipError_t launch_mxfp4_quant(const Shape& s, const void* q, const void* k, const float* k_mean,
                              void* workspace, hipStream_t stream);
Fp4Codes fp4_codes(void* workspace, const Shape& s);

// Most key blocks (N / 64) the pattern prediction supports.
int pattern_max_nkb();

// Vertical / slash lines of every (b, hq) from the votes of its kept lists
// (lines [B*Hq][n_vertical + n_slash]) and the lists extended by them.
hipError_t launch_patterns(const Shape& s, const int32_t* kv_idx, const int32_t* kv_cnt,
                           int max_keep, int n_vertical, int n_slash, int32_t* kv_idx_out,
                           int32_t* kv_cnt_out, int max_keep_out, int32_t* lines,
                           hipStream_t stream);

// Longest key list the gathered-key forward accepts (entries per query block).
int fwd_max_gather_keys();

// Anchor-based stripe selection: key lists [B*Hq*nqb][max_keys] and counts.
hipError_t launch_stripe_select(const Shape& s, const float* q_pool, const int8_t* k_i8,
                                const float* k_scale, float theta, int max_keys,
                                int32_t* key_idx, int32_t* key_cnt, hipStream_t stream);

// Per-head sampled RMS logit error of the INT8 path against the 16-bit path;
// head_hi (optional) gets err > threshold.
hipError_t launch_head_error(const Shape& s, const int8_t* q_i8, const float* q_scale,
                             const int8_t* k_i8, const float* k_scale, const void* q,
                             const void* k, const float* k_mean, float threshold,
                             float* head_err, int32_t* head_hi, hipStream_t stream);

}  // namespace qattn
