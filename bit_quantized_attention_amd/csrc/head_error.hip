// Per-head error proxy of the INT8 Q K^T (adaptive per-head precision).
//
// One 4-wave workgroup per (b, hq). Over a fixed sample of up to 64 query rows
// (one per evenly spaced query block) and up to 256 keys (one per evenly
// spaced key block), every (row, key) pair is scored twice on the matrix
// cores: the INT8 path's base-2 logit s8 = fl32(S * alpha), with S the exact
// code product (v_mfma_i32_32x32x32_i8) and alpha = fl32(fl32(sq * c) * sk),
// and the 16-bit path's logit s16 = c * (q . k - q . k_mean)
// (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation). The head's error is
// sqrt(mean (s8 - s16)^2); heads above the caller's threshold are flagged for
// 16-bit Q K^T.
//
// Layout: wave w takes sampled rows 32*(w%2) + [0, 32) as the 32 columns of
// its MFMA blocks and the key blocks w/2, w/2+2, w/2+4, w/2+6 of 32 sampled
// keys each. Fragments come straight from global memory (the sample is
// scattered and read once). The sums are reduced in a fixed order, so the
// result does not depend on timing.
#include "../../include/qattn.h"
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kMaxRows = 64;
constexpr int kMaxKeys = 256;

struct HeArgs {
  const int8_t* q_i8;
  const float* q_scale;
  const int8_t* k_i8;
  const float* k_scale;
  const uint16_t* q16;
  const uint16_t* k16;
  const float* k_mean;
  float* head_err;
  int32_t* head_hi;
  float threshold;
  float c;  // fl32(log2(e) / sqrt(d))
  int Hq, Hkv, N, group, nqb, nkb, nsq, nsk;
};

template <bool BF16>
struct Op16;
template <>
struct Op16<true> {
  typedef v8bf t;
  typedef __bf16 el;
  static __device__ __forceinline__ v16f mma(t a, t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Op16<false> {
  typedef v8h t;
  typedef _Float16 el;
  static __device__ __forceinline__ v16f mma(t a, t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// sampled query row u of nsq (query block floor(u * nqb / nsq), fixed offset)
__device__ __forceinline__ int sample_row(int u, int nqb, int nsq) {
  return kQBlock * (int)(((long long)u * nqb) / nsq) + (37 * u + 11) % kQBlock;
}
// sampled key w of nsk (key block floor(w * nkb / nsk), fixed offset)
__device__ __forceinline__ int sample_key_block(int w, int nkb, int nsk) {
  return (int)(((long long)w * nkb) / nsk);
}
__device__ __forceinline__ int sample_key(int w, int nkb, int nsk) {
  return kKBlock * sample_key_block(w, nkb, nsk) + (29 * w + 5) % kKBlock;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void head_error_kernel(HeArgs a) {
  using O = Op16<BF16>;
  typedef typename O::t op_t;
  constexpr int KS8 = D / 32;   // 32-deep k-steps of the INT8 product
  constexpr int KS16 = D / 16;  // 16-deep k-steps of the 16-bit product
  __shared__ float wsum[4];
  const int bhq = blockIdx.x;
  const int b = bhq / a.Hq;
  const int hq = bhq % a.Hq;
  const int kvu = b * a.Hkv + hq / a.group;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // this lane's query column: sampled row u (a valid row is loaded for the
  // padding columns u >= nsq, whose pairs are not counted)
  const int u = 32 * (wave & 1) + l32;
  const bool q_ok = u < a.nsq;
  const int row = sample_row(q_ok ? u : 0, a.nqb, a.nsq);
  const int8_t* q8 = a.q_i8 + ((size_t)bhq * a.N + row) * D;
  const uint16_t* qh = a.q16 + ((size_t)bhq * a.N + row) * D;
  v4i qf[KS8];
  op_t qf16[KS16];
#pragma unroll
  for (int ks = 0; ks < KS8; ++ks) qf[ks] = *reinterpret_cast<const v4i*>(q8 + 32 * ks + 16 * h);
#pragma unroll
  for (int ks = 0; ks < KS16; ++ks) qf16[ks] = *reinterpret_cast<const op_t*>(qh + 16 * ks + 8 * h);
  // q . k_mean over the row (each lane half holds half of the channels)
  const float* mean = a.k_mean + (size_t)kvu * D;
  float part = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS16; ++ks) {
    const float4 m0 = *reinterpret_cast<const float4*>(mean + 16 * ks + 8 * h);
    const float4 m1 = *reinterpret_cast<const float4*>(mean + 16 * ks + 8 * h + 4);
    const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qf16[ks][e], mv[e], part);
  }
  const float qm = part + __shfl_xor(part, 32, 64);
  const float alpha_q = a.q_scale[(size_t)bhq * a.nqb + row / kQBlock] * a.c;

  float sum = 0.0f;
  for (int i = 0; i < 4; ++i) {
    const int kb = (wave >> 1) + 2 * i;  // block of 32 sampled keys
    if (32 * kb >= a.nsk) break;         // uniform over the wave
    // A operand: sampled key 32*kb + l32 (padding lanes load key 0's row)
    const int wk = 32 * kb + l32;
    const bool k_ok = wk < a.nsk;
    const int key = sample_key(k_ok ? wk : 0, a.nkb, a.nsk);
    const int8_t* k8 = a.k_i8 + ((size_t)kvu * a.N + key) * D;
    const uint16_t* kh = a.k16 + ((size_t)kvu * a.N + key) * D;
    const float kscale_row =
        a.k_scale[(size_t)kvu * a.nkb + sample_key_block(k_ok ? wk : 0, a.nkb, a.nsk)];
    v16i si;
    v16f sh;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      si[r] = 0;
      sh[r] = 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      const v4i kf = *reinterpret_cast<const v4i*>(k8 + 32 * ks + 16 * h);
      si = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[ks], si, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks) {
      const op_t kf = *reinterpret_cast<const op_t*>(kh + 16 * ks + 8 * h);
      sh = O::mma(kf, qf16[ks], sh);
    }
    // element r holds key row kr = 8*(r/4) + 4*h + r%4 of the block, query l32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * h + (r & 3);
      const float sk = __shfl(kscale_row, kr, 64);
      const float alpha = alpha_q * sk;
      const float s8 = (float)(int)si[r] * alpha;
      const float s16 = a.c * (sh[r] - qm);
      const float e = s8 - s16;
      if (q_ok && 32 * kb + kr < a.nsk) sum = __builtin_fmaf(e, e, sum);
    }
  }
  // fixed-order reduction: butterfly within the wave, then the four waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane == 0) wsum[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const float err = __builtin_sqrtf(tot / (float)(a.nsq * a.nsk));
    a.head_err[bhq] = err;
    if (a.head_hi != nullptr) a.head_hi[bhq] = err > a.threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_head_error(const Shape& s, const int8_t* q_i8, const float* q_scale,
                             const int8_t* k_i8, const float* k_scale, const void* q,
                             const void* k, const float* k_mean, float threshold,
                             float* head_err, int32_t* head_hi, hipStream_t stream) {
  HeArgs a;
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.q16 = static_cast<const uint16_t*>(q);
  a.k16 = static_cast<const uint16_t*>(k);
  a.k_mean = k_mean;
  a.head_err = head_err;
  a.head_hi = head_hi;
  a.threshold = threshold;
  a.c = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d));
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.group = s.Hq / s.Hkv;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.nsq = a.nqb < kMaxRows ? a.nqb : kMaxRows;
  a.nsk = a.nkb < kMaxKeys ? a.nkb : kMaxKeys;
  const dim3 grid(s.B * s.Hq);
  if (s.d == 128) {
    if (s.bf16) hipLaunchKernelGGL((head_error_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((head_error_kernel<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (s.bf16) hipLaunchKernelGGL((head_error_kernel<64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((head_error_kernel<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qattn
