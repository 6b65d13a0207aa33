// C ABI of the qattn library: host-side validation, then the kernel launchers.
// Every check happens before the first HIP call; no exception leaves this file.
#include "../../include/qattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "qattn_internal.h"

namespace {

using qattn::Shape;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

qattn_status_t check_problem(const qattn_problem_t* p, Shape* s) {
  if (p == nullptr) return QATTN_ERR_NULL;
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->N <= 0 || p->d <= 0) return QATTN_ERR_SHAPE;
  if (p->Hq % p->Hkv != 0) return QATTN_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return QATTN_ERR_UNSUPPORTED;
  if (p->N % QATTN_Q_BLOCK != 0) return QATTN_ERR_UNSUPPORTED;
  if (p->dtype != QATTN_F16 && p->dtype != QATTN_BF16) return QATTN_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return QATTN_ERR_ARG;
  // element offsets and token indices stay within the integer types used in
  // the kernels (64-bit element offsets, 32-bit tokens and block indices)
  const long long rows = (long long)p->B * p->Hq * p->N;
  if (rows > (1LL << 40)) return QATTN_ERR_UNSUPPORTED;
  s->B = p->B;
  s->Hq = p->Hq;
  s->Hkv = p->Hkv;
  s->N = p->N;
  s->d = p->d;
  s->bf16 = p->dtype == QATTN_BF16 ? 1 : 0;
  s->causal = p->causal;
  return QATTN_OK;
}

bool ratio_ok(int32_t num, int32_t den) { return den > 0 && num >= 0 && num <= den; }

int32_t max_keep_of(const Shape& s, int32_t num, int32_t den) {
  const long long nkb = s.nkb();
  long long k = 3 + (nkb * num + den - 1) / den;
  if (k > nkb) k = nkb;
  return (int32_t)k;
}

qattn_status_t launched(hipError_t e) { return e == hipSuccess ? QATTN_OK : QATTN_ERR_DEVICE; }

// Both preprocessing calls share one workspace of this size.
size_t workspace_of(const Shape& s) {
  const size_t a = qattn::ksum_workspace_bytes(s);
  const size_t b = qattn::mask_workspace_bytes(s);
  return a > b ? a : b;
}

}  // namespace

extern "C" {

const char* qattn_status_str(qattn_status_t status) {
  switch (status) {
    case QATTN_OK: return "ok";
    case QATTN_ERR_NULL: return "a required pointer is NULL";
    case QATTN_ERR_SHAPE: return "invalid shape (a dimension <= 0, or Hq not a multiple of Hkv)";
    case QATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case QATTN_ERR_UNSUPPORTED:
      return "unsupported problem (d must be 64 or 128, N a multiple of 128, dtype f16/bf16)";
    case QATTN_ERR_ARG: return "invalid argument (flag, keep ratio, max_keep or workspace size)";
    case QATTN_ERR_DEVICE: return "HIP launch failed";
    case QATTN_ERR_SCRATCH:
      return "the problem needs more scratch than the allocation-free entry point's static array";
  }
  return "unknown status";
}

const char* qattn_version(void) { return "qattn 0.1.0 gfx950"; }

size_t qattn_workspace_bytes(const qattn_problem_t* p) {
  Shape s;
  if (check_problem(p, &s) != QATTN_OK) return 0;
  return workspace_of(s);
}

int32_t qattn_max_keep(const qattn_problem_t* p, int32_t keep_num, int32_t keep_den) {
  Shape s;
  if (check_problem(p, &s) != QATTN_OK || !ratio_ok(keep_num, keep_den)) return -1;
  return max_keep_of(s, keep_num, keep_den);
}

qattn_status_t qattn_smooth_quant(const qattn_problem_t* p, const void* q, const void* k,
                                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                  float* k_mean, float* q_pool, float* k_pool, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean || !workspace)
    return QATTN_ERR_NULL;
  const void* ptrs[] = {q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool, workspace};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (workspace_bytes < workspace_of(s)) return QATTN_ERR_ARG;
  return launched(qattn::launch_smooth_quant(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool,
                                             k_pool, workspace,
                                             static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_smooth_quant_noalloc(const qattn_problem_t* p, const void* q, const void* k,
                                          int8_t* q_i8, float* q_scale, int8_t* k_i8,
                                          float* k_scale, float* k_mean, float* q_pool,
                                          float* k_pool, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean) return QATTN_ERR_NULL;
  const void* ptrs[] = {q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (qattn::ksum_workspace_bytes(s) > qattn::kNoallocScratchBytes) return QATTN_ERR_SCRATCH;
  return launched(qattn::launch_smooth_quant_noalloc(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean,
                                                     q_pool, k_pool,
                                                     static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_block_mask(const qattn_problem_t* p, const float* q_pool, const float* k_pool,
                                int32_t keep_num, int32_t keep_den, int32_t max_keep,
                                int32_t* kv_idx, int32_t* kv_cnt, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::mask_max_nkb()) return QATTN_ERR_UNSUPPORTED;
  if (!q_pool || !k_pool || !kv_idx || !kv_cnt || !workspace) return QATTN_ERR_NULL;
  const void* ptrs[] = {q_pool, k_pool, kv_idx, kv_cnt, workspace};
  for (const void* x : ptrs)
    if (misaligned(x)) return QATTN_ERR_ALIGN;
  if (!ratio_ok(keep_num, keep_den)) return QATTN_ERR_ARG;
  if (max_keep < max_keep_of(s, keep_num, keep_den)) return QATTN_ERR_ARG;
  if (workspace_bytes < workspace_of(s)) return QATTN_ERR_ARG;
  return launched(qattn::launch_block_mask(s, q_pool, k_pool, keep_num, keep_den, max_keep, kv_idx,
                                           kv_cnt, workspace, static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_fwd(const qattn_problem_t* p, const int8_t* q_i8, const float* q_scale,
                         const int8_t* k_i8, const float* k_scale, const void* v,
                         const int32_t* kv_idx, const int32_t* kv_cnt, int32_t max_keep, void* o,
                         float* lse, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v || !o) return QATTN_ERR_NULL;
  const void* ptrs[] = {q_i8, q_scale, k_i8, k_scale, v, o, lse, kv_idx, kv_cnt};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if ((kv_idx == nullptr) != (kv_cnt == nullptr)) return QATTN_ERR_ARG;
  // a kept list indexes at most fwd_max_sparse_tiles() 64-key blocks (N <= 131072)
  if (kv_idx != nullptr && s.nkb() > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_UNSUPPORTED;
  if (kv_idx != nullptr && (max_keep < 1 || max_keep > qattn::fwd_max_sparse_tiles()))
    return QATTN_ERR_ARG;
  return launched(qattn::launch_attn_fwd(s, q_i8, q_scale, k_i8, k_scale, v, kv_idx, kv_cnt,
                                         max_keep, nullptr, nullptr, nullptr, nullptr, false, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_fwd_promoted(const qattn_problem_t* p, const int8_t* q_i8,
                                  const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                  const void* q, const void* k, const float* k_mean,
                                  const void* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                                  int32_t max_keep, void* o, float* lse, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_UNSUPPORTED;
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !q || !k || !k_mean || !v || !kv_idx ||
      !kv_cnt || !o)
    return QATTN_ERR_NULL;
  const void* ptrs[] = {q_i8, q_scale, k_i8, k_scale, q, k, k_mean, v, kv_idx, kv_cnt, o, lse};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (max_keep < 1 || max_keep > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_ARG;
  return launched(qattn::launch_attn_fwd(s, q_i8, q_scale, k_i8, k_scale, v, kv_idx, kv_cnt,
                                         max_keep, q, k, k_mean, nullptr, false, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_fwd_promoted_fp4(const qattn_problem_t* p, const void* q, const void* k,
                                      const float* k_mean, const void* v, const int32_t* kv_idx,
                                      const int32_t* kv_cnt, int32_t max_keep, void* o, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_UNSUPPORTED;
  if (!q || !k || !k_mean || !v || !kv_idx || !kv_cnt || !o || !workspace) return QATTN_ERR_NULL;
  const void* ptrs[] = {q, k, k_mean, v, kv_idx, kv_cnt, o, lse, workspace};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (max_keep < 1 || max_keep > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_ARG;
  if (workspace_bytes < qattn::lowbit_workspace_bytes(s, false)) return QATTN_ERR_ARG;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = qattn::launch_mxfp4_quant(s, q, k, k_mean, workspace, hs);
  if (e != hipSuccess) return QATTN_ERR_DEVICE;
  const qattn::Fp4Codes codes = qattn::fp4_codes(workspace, s);
  return launched(qattn::launch_attn_fwd(s, nullptr, nullptr, nullptr, nullptr, v, kv_idx, kv_cnt,
                                         max_keep, q, k, k_mean, nullptr, false, o, lse, hs,
                                         &codes));
}

size_t qattn_lowbit_workspace_bytes(const qattn_problem_t* p) {
  Shape s;
  if (check_problem(p, &s) != QATTN_OK) return 0;
  return qattn::lowbit_workspace_bytes(s, true);
}

qattn_status_t qattn_block_mask_lowbit(const qattn_problem_t* p, const void* q, const void* k,
                                       const float* k_mean, int32_t keep_num, int32_t keep_den,
                                       int32_t max_keep, int32_t* kv_idx, int32_t* kv_cnt,
                                       float* scores, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::mask_max_nkb()) return QATTN_ERR_UNSUPPORTED;
  if (!q || !k || !k_mean || !kv_idx || !kv_cnt || !workspace) return QATTN_ERR_NULL;
  const void* ptrs[] = {q, k, k_mean, kv_idx, kv_cnt, scores, workspace};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (!ratio_ok(keep_num, keep_den)) return QATTN_ERR_ARG;
  if (max_keep < max_keep_of(s, keep_num, keep_den)) return QATTN_ERR_ARG;
  if (workspace_bytes < qattn::lowbit_workspace_bytes(s, true)) return QATTN_ERR_ARG;
  return launched(qattn::launch_lowbit_mask(s, q, k, k_mean, keep_num, keep_den, max_keep, kv_idx,
                                            kv_cnt, scores, workspace,
                                            static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_block_mask_patterns(const qattn_problem_t* p, const int32_t* kv_idx,
                                         const int32_t* kv_cnt, int32_t max_keep,
                                         int32_t n_vertical, int32_t n_slash, int32_t* kv_idx_out,
                                         int32_t* kv_cnt_out, int32_t max_keep_out,
                                         int32_t* lines, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::pattern_max_nkb()) return QATTN_ERR_UNSUPPORTED;
  if (!kv_idx || !kv_cnt || !kv_idx_out || !kv_cnt_out) return QATTN_ERR_NULL;
  if (n_vertical + n_slash > 0 && !lines) return QATTN_ERR_NULL;
  const void* ptrs[] = {kv_idx, kv_cnt, kv_idx_out, kv_cnt_out, lines};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (n_vertical < 0 || n_vertical > QATTN_MAX_PATTERN_LINES || n_slash < 0 ||
      n_slash > QATTN_MAX_PATTERN_LINES)
    return QATTN_ERR_ARG;
  if (max_keep < 1) return QATTN_ERR_ARG;
  const long long need = std::min<long long>(s.nkb(), (long long)max_keep + n_vertical + n_slash);
  if (max_keep_out < need) return QATTN_ERR_ARG;
  // the outputs are written while other rows' inputs are still read
  const size_t rows = (size_t)s.B * s.Hq * s.nqb();
  const auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
  };
  const size_t in_b = rows * (size_t)max_keep * 4, out_b = rows * (size_t)max_keep_out * 4;
  if (overlap(kv_idx, in_b, kv_idx_out, out_b) || overlap(kv_cnt, rows * 4, kv_cnt_out, rows * 4) ||
      overlap(kv_idx, in_b, kv_cnt_out, rows * 4) || overlap(kv_cnt, rows * 4, kv_idx_out, out_b))
    return QATTN_ERR_ARG;
  return launched(qattn::launch_patterns(s, kv_idx, kv_cnt, max_keep, n_vertical, n_slash,
                                         kv_idx_out, kv_cnt_out, max_keep_out, lines,
                                         static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_stripe_select(const qattn_problem_t* p, const float* q_pool,
                                   const int8_t* k_i8, const float* k_scale, float theta,
                                   int32_t max_keys, int32_t* key_idx, int32_t* key_cnt,
                                   void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.N > 65536) return QATTN_ERR_UNSUPPORTED;
  if (!q_pool || !k_i8 || !k_scale || !key_idx || !key_cnt) return QATTN_ERR_NULL;
  const void* ptrs[] = {q_pool, k_i8, k_scale, key_idx, key_cnt};
  for (const void* x : ptrs)
    if (misaligned(x)) return QATTN_ERR_ALIGN;
  if (std::isnan(theta)) return QATTN_ERR_ARG;
  // the anchor region (up to 64 + 128 keys) always fits
  if (max_keys < QATTN_K_BLOCK + QATTN_Q_BLOCK || max_keys > qattn::fwd_max_gather_keys())
    return QATTN_ERR_ARG;
  return launched(qattn::launch_stripe_select(s, q_pool, k_i8, k_scale, theta, max_keys, key_idx,
                                              key_cnt, static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_fwd_stripes(const qattn_problem_t* p, const int8_t* q_i8,
                                 const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                 const void* v, const int32_t* key_idx, const int32_t* key_cnt,
                                 int32_t max_keys, void* o, float* lse, void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.N > 65536) return QATTN_ERR_UNSUPPORTED;
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v || !key_idx || !key_cnt || !o)
    return QATTN_ERR_NULL;
  const void* ptrs[] = {q_i8, q_scale, k_i8, k_scale, v, key_idx, key_cnt, o, lse};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (max_keys < 1 || max_keys > qattn::fwd_max_gather_keys()) return QATTN_ERR_ARG;
  return launched(qattn::launch_attn_fwd(s, q_i8, q_scale, k_i8, k_scale, v, key_idx, key_cnt,
                                         max_keys, nullptr, nullptr, nullptr, nullptr, true, o,
                                         lse, static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_head_error(const qattn_problem_t* p, const int8_t* q_i8,
                                const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                const void* q, const void* k, const float* k_mean,
                                float threshold, float* head_err, int32_t* head_hi,
                                void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !q || !k || !k_mean || !head_err)
    return QATTN_ERR_NULL;
  const void* ptrs[] = {q_i8, q_scale, k_i8, k_scale, q, k, k_mean, head_err, head_hi};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  if (!(threshold >= 0.0f) || !std::isfinite(threshold)) return QATTN_ERR_ARG;
  return launched(qattn::launch_head_error(s, q_i8, q_scale, k_i8, k_scale, q, k, k_mean,
                                           threshold, head_err, head_hi,
                                           static_cast<hipStream_t>(stream)));
}

qattn_status_t qattn_fwd_adaptive(const qattn_problem_t* p, const int8_t* q_i8,
                                  const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                  const void* q, const void* k, const float* k_mean,
                                  const void* v, const int32_t* head_hi, void* o, float* lse,
                                  void* stream) {
  Shape s;
  const qattn_status_t st = check_problem(p, &s);
  if (st != QATTN_OK) return st;
  if (s.nkb() > qattn::fwd_max_sparse_tiles()) return QATTN_ERR_UNSUPPORTED;
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !q || !k || !k_mean || !v || !head_hi || !o)
    return QATTN_ERR_NULL;
  const void* ptrs[] = {q_i8, q_scale, k_i8, k_scale, q, k, k_mean, v, head_hi, o, lse};
  for (const void* x : ptrs)
    if (x && misaligned(x)) return QATTN_ERR_ALIGN;
  return launched(qattn::launch_attn_fwd(s, q_i8, q_scale, k_i8, k_scale, v, nullptr, nullptr, 0,
                                         q, k, k_mean, head_hi, false, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
