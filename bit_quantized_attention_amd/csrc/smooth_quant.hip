// K smoothing and per-block INT8 quantization of Q and K (bandwidth-bound).
//
// Three launches on the caller's stream:
//   1. ksum_qquant    -- exact per-channel sums of K over 128-token chunks
//                        (fp64 double-double), one workgroup per (chunk, b*hk),
//                        then one workgroup per Q block (128 tokens): amax,
//                        scale, exact RNE codes, optional pooled block means;
//   2. kmean_finalize -- merge the chunks, k_mean = fl32(fl64(sum) / N);
//   3. kquant         -- one workgroup per K block (64 tokens), smoothed by
//                        k_mean, as for Q.
// Every element is read with 16-byte vector loads; a 64-lane wave covers 4
// (d = 128) or 8 (d = 64) contiguous rows per load instruction.
#include "device_util.h"
#include "qattn_internal.h"

#include <mutex>

// The rounding sequence of every value here is fixed by the definition: no
// contraction of a*b+c into fma anywhere in this file.
#pragma clang fp contract(off)

namespace qattn {
namespace {

constexpr int kThreads = 256;

// Exact per-channel sums of K over one chunk of kKsumChunk tokens of head bh.
template <int D, bool BF16>
__device__ __forceinline__ void ksum_chunk(const uint16_t* __restrict__ k,
                                           double2* __restrict__ part, int N, int nchunk,
                                           int chunk, int bh, double2 (*red)[D]) {
  constexpr int LPR = D / 8;          // lanes per row (16 bytes each)
  constexpr int RPI = kThreads / LPR; // rows per iteration
  const int cg = threadIdx.x % LPR;
  const int rg = threadIdx.x / LPR;
  const int t0 = chunk * kKsumChunk;
  const int t1 = min(N, t0 + kKsumChunk);
  const uint16_t* base = k + (size_t)bh * N * D + cg * 8;
  double hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) hi[e] = lo[e] = 0.0;
  for (int t = t0 + rg; t < t1; t += RPI) {
    float x[8];
    load8_f32<BF16>(base + (size_t)t * D, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) dd_add(hi[e], lo[e], (double)x[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = make_double2(hi[e], lo[e]);
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    double H = 0.0, L = 0.0;
    for (int r = 0; r < RPI; ++r) dd_merge(H, L, red[r][c].x, red[r][c].y);
    part[((size_t)bh * nchunk + chunk) * D + c] = make_double2(H, L);
  }
}

// One workgroup of kFinGroups x kFinChans threads per (b, hk, slice of
// kFinChans channels): group g merges chunks g, g + kFinGroups, ... of its
// channel (four loads in flight), then the groups merge pairwise in LDS. The
// double-double sums are exact for any realistic K, so the order is free.
constexpr int kFinGroups = 32;
constexpr int kFinChans = 32;

__global__ __launch_bounds__(kFinGroups * kFinChans) void kmean_finalize_kernel(
    const double2* __restrict__ part, float* __restrict__ k_mean, int N, int nchunk, int D) {
  __shared__ double2 red[kFinGroups][kFinChans];
  const int bh = blockIdx.x;
  const int cs = threadIdx.x % kFinChans;
  const int g = threadIdx.x / kFinChans;
  const int c = blockIdx.y * kFinChans + cs;
  const double2* src = part + (size_t)bh * nchunk * D + c;
  double H = 0.0, L = 0.0;
  int ch = g;
  for (; ch + 3 * kFinGroups < nchunk; ch += 4 * kFinGroups) {
    double2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[(size_t)(ch + u * kFinGroups) * D];
#pragma unroll
    for (int u = 0; u < 4; ++u) dd_merge(H, L, v[u].x, v[u].y);
  }
  for (; ch < nchunk; ch += kFinGroups) {
    const double2 v = src[(size_t)ch * D];
    dd_merge(H, L, v.x, v.y);
  }
  red[g][cs] = make_double2(H, L);
#pragma unroll
  for (int w = kFinGroups / 2; w >= 1; w /= 2) {
    __syncthreads();
    if (g < w) {
      const double2 o = red[g + w][cs];
      dd_merge(H, L, o.x, o.y);
      red[g][cs] = make_double2(H, L);
    }
  }
  if (g == 0) {
    const double sum = H + L;  // the fp64 value nearest the exact sum
    k_mean[(size_t)bh * D + c] = (float)(sum / (double)N);
  }
}

struct QuantArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* k_mean;
  int8_t* q_i8;
  float* q_scale;
  int8_t* k_i8;
  float* k_scale;
  float* q_pool;
  float* k_pool;
  int N;
  int nQ;   // number of Q blocks = B*Hq*nqb
  int nqb;
  int nkb;
};

// One block of ROWS tokens x D channels: src/dst point at its first row.
template <int D, bool BF16, int ROWS, bool IS_K>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ src,
                                            const float* __restrict__ mean,
                                            int8_t* __restrict__ dst, float* scale_out,
                                            float* __restrict__ pool_out,
                                            double2 (*red)[D], float* wmax) {
  constexpr int LPR = D / 8;
  constexpr int RPI = kThreads / LPR;
  constexpr int RPT = ROWS / RPI;  // rows per thread
  const int cg = threadIdx.x % LPR;
  const int rg = threadIdx.x / LPR;
  float x[RPT][8];
#pragma unroll
  for (int i = 0; i < RPT; ++i) load8_f32<BF16>(src + (size_t)(rg + i * RPI) * D + cg * 8, x[i]);

  if (pool_out != nullptr) {
    // exact column sums of the raw 16-bit values
    double hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hi[e] = lo[e] = 0.0;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) dd_add(hi[e], lo[e], (double)x[i][e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = make_double2(hi[e], lo[e]);
  }

  float m[8];
  if constexpr (IS_K) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = mean[cg * 8 + e];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] - m[e];
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i][e]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
  const float scale = quant_scale(amax);
  const float inv = 1.0f / scale;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    uint2 w;
    w.x = pack4_i8(quant_code(x[i][0], scale, inv), quant_code(x[i][1], scale, inv),
                   quant_code(x[i][2], scale, inv), quant_code(x[i][3], scale, inv));
    w.y = pack4_i8(quant_code(x[i][4], scale, inv), quant_code(x[i][5], scale, inv),
                   quant_code(x[i][6], scale, inv), quant_code(x[i][7], scale, inv));
    *reinterpret_cast<uint2*>(dst + (size_t)(rg + i * RPI) * D + cg * 8) = w;
  }
  if (threadIdx.x == 0) *scale_out = scale;

  if (pool_out != nullptr && threadIdx.x < D) {
    const int c = threadIdx.x;
    double H = 0.0, L = 0.0;
    for (int r = 0; r < RPI; ++r) dd_merge(H, L, red[r][c].x, red[r][c].y);
    const double s = H + L;
    if constexpr (IS_K) {
      pool_out[c] = (float)(s / (double)ROWS - (double)mean[c]);
    } else {
      pool_out[c] = (float)(s / (double)ROWS);
    }
  }
}

// Pass 1: the K chunk sums (first, so that the finalize can start early) and
// every Q block, which does not depend on the K mean.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void ksum_qquant_kernel(QuantArgs a, double2* part,
                                                               int nchunk, int nsum) {
  constexpr int RPI = kThreads / (D / 8);
  __shared__ double2 red[RPI][D];
  __shared__ float wmax[kThreads / 64];
  const int blk = blockIdx.x;
  if (blk < nsum) {
    ksum_chunk<D, BF16>(a.k, part, a.N, nchunk, blk % nchunk, blk / nchunk, red);
    return;
  }
  const int qblk = blk - nsum;
  const size_t bh = qblk / a.nqb;  // b * Hq + hq
  const int i = qblk % a.nqb;
  const size_t row0 = bh * a.N + (size_t)i * kQBlock;
  quant_block<D, BF16, kQBlock, false>(a.q + row0 * D, nullptr, a.q_i8 + row0 * D,
                                       a.q_scale + qblk,
                                       a.q_pool ? a.q_pool + (size_t)qblk * D : nullptr, red,
                                       wmax);
}

// Pass 3: every K block, smoothed by the finished K mean.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void kquant_kernel(QuantArgs a) {
  constexpr int RPI = kThreads / (D / 8);
  __shared__ double2 red[RPI][D];
  __shared__ float wmax[kThreads / 64];
  const int kblk = blockIdx.x;
  const size_t bh = kblk / a.nkb;  // b * Hkv + hk
  const int j = kblk % a.nkb;
  const size_t row0 = bh * a.N + (size_t)j * kKBlock;
  quant_block<D, BF16, kKBlock, true>(a.k + row0 * D, a.k_mean + bh * D, a.k_i8 + row0 * D,
                                      a.k_scale + kblk,
                                      a.k_pool ? a.k_pool + (size_t)kblk * D : nullptr, red,
                                      wmax);
}

template <int D, bool BF16>
hipError_t launch(const Shape& s, const void* q, const void* k, int8_t* q_i8, float* q_scale,
                  int8_t* k_i8, float* k_scale, float* k_mean, float* q_pool, float* k_pool,
                  void* workspace, hipStream_t stream) {
  const int nchunk = s.nchunk();
  double2* part = static_cast<double2*>(workspace);
  QuantArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.k_mean = k_mean;
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.q_pool = q_pool;
  a.k_pool = k_pool;
  a.N = s.N;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.nQ = s.B * s.Hq * a.nqb;
  const int nsum = s.B * s.Hkv * nchunk;
  const int nK = s.B * s.Hkv * a.nkb;
  hipLaunchKernelGGL((ksum_qquant_kernel<D, BF16>), dim3(nsum + a.nQ), dim3(kThreads), 0, stream,
                     a, part, nchunk, nsum);
  hipLaunchKernelGGL(kmean_finalize_kernel, dim3(s.B * s.Hkv, D / kFinChans),
                     dim3(kFinGroups * kFinChans), 0, stream, part, k_mean, s.N, nchunk, D);
  hipLaunchKernelGGL((kquant_kernel<D, BF16>), dim3(nK), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// The allocation-free entry point's partial sums: a file-scope device array,
// one copy per GPU. Host code never passes its name to a kernel (on the host
// the name is a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The scratch address of the current device, looked up on the device's first
// call (with the device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_smooth_quant_noalloc(const Shape& s, const void* q, const void* k, int8_t* q_i8,
                                       float* q_scale, int8_t* k_i8, float* k_scale,
                                       float* k_mean, float* q_pool, float* k_pool,
                                       hipStream_t stream) {
  if (ksum_workspace_bytes(s) > kNoallocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  // every partial sum is written by the first launch before the second reads
  // it, so nothing needs clearing
  return launch_smooth_quant(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool, ws,
                             stream);
}

hipError_t launch_smooth_quant(const Shape& s, const void* q, const void* k, int8_t* q_i8,
                               float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                               float* q_pool, float* k_pool, void* workspace,
                               hipStream_t stream) {
  if (s.d == 128) {
    return s.bf16 ? launch<128, true>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool,
                                      k_pool, workspace, stream)
                  : launch<128, false>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool,
                                       k_pool, workspace, stream);
  }
  return s.bf16 ? launch<64, true>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool,
                                   workspace, stream)
                : launch<64, false>(s, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool,
                                    workspace, stream);
}

}  // namespace qattn
