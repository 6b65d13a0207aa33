// Anchor-based stripe selection: per (b, hq, query block), the key positions
// whose score comes within a threshold of the anchor.
//
// One 4-wave workgroup per (b, kv head, query block); wave w takes query heads
// w, w+4, ... of the group. A wave INT8-quantizes its block's mean query (the
// pooled-mask rule), scores the anchor region (the first 64 keys and the
// block's own 128 positions) straight from global memory to find the anchor,
// then scores every causally valid key against fl32(anchor - theta): chunks
// of 256 key code rows are staged in LDS once per workgroup and scored with
// v_dot4 (exact int32, then two fp32 roundings). Ballot prefix counts write
// the kept keys in ascending order; past the capacity only the anchor region
// is still written.
#include "device_util.h"
#include "qattn_internal.h"

#pragma clang fp contract(off)

namespace qattn {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;

struct StripeArgs {
  const float* q_pool;
  const int8_t* k_i8;
  const float* k_scale;
  int32_t* key_idx;
  int32_t* key_cnt;
  float theta;
  int B, Hq, Hkv, group, N, nqb, nkb, causal, max_keys;
};

template <int D>
__device__ __forceinline__ float key_score(const int32_t (&qw)[D / 4], const int8_t* krow,
                                           float qs, float ks) {
  int dot = 0;
#pragma unroll
  for (int w4 = 0; w4 < D / 16; ++w4) {
    const int4 kk = *reinterpret_cast<const int4*>(krow + 16 * w4);
    dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 0], kk.x, dot, false);
    dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 1], kk.y, dot, false);
    dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 2], kk.z, dot, false);
    dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 3], kk.w, dot, false);
  }
  const float s1 = (float)dot * qs;
  return s1 * ks;
}

template <int D>
__global__ __launch_bounds__(kThreads) void stripe_select_kernel(StripeArgs a) {
  constexpr int KSTR = D + 16;  // padded LDS rows: 16-byte reads of 8 rows hit distinct banks
  __shared__ __attribute__((aligned(16))) int8_t kcodes[kChunk * KSTR];
  __shared__ __attribute__((aligned(16))) int8_t qcodes[4][D];
  __shared__ float qscale[4];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // longest causal rows first
  const int slot = blockIdx.x % (a.B * a.Hkv);
  const int rank = blockIdx.x / (a.B * a.Hkv);
  const int i = a.causal ? a.nqb - 1 - rank : rank;
  const int b = slot / a.Hkv;
  const int hk = slot % a.Hkv;
  const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.N;
  const float* kscale = a.k_scale + ((size_t)b * a.Hkv + hk) * a.nkb;
  const int nvis = a.causal ? min(a.N, kQBlock * i + kQBlock) : a.N;
  const int loc0 = kQBlock * i;  // local window [loc0, loc0 + 128)
  auto in_region = [&](int k) { return k < kKBlock || (k >= loc0 && k < loc0 + kQBlock); };
  const int nregion = min(kKBlock, nvis) + max(0, min(nvis, loc0 + kQBlock) - max(loc0, kKBlock));
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rounds = (a.group + 3) / 4;

  for (int round = 0; round < rounds; ++round) {
    const int g = round * 4 + wave;
    const bool active = g < a.group;  // wave-uniform
    const int hq = hk * a.group + (active ? g : 0);
    const size_t row = ((size_t)b * a.Hq + hq) * a.nqb + i;
    // the mean query's INT8 codes (8 channels per lane on D/8 lanes)
    if (active) {
      constexpr int LPV = D / 8;
      const int sub = lane % LPV;
      float v[8];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = a.q_pool[row * D + sub * 8 + e];
        am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
      }
#pragma unroll
      for (int o = LPV / 2; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o, 64));
      const float s = quant_scale(am);
      const float inv = 1.0f / s;
      if (lane < LPV) {
        uint2 w;
        w.x = pack4_i8(quant_code(v[0], s, inv), quant_code(v[1], s, inv), quant_code(v[2], s, inv),
                       quant_code(v[3], s, inv));
        w.y = pack4_i8(quant_code(v[4], s, inv), quant_code(v[5], s, inv), quant_code(v[6], s, inv),
                       quant_code(v[7], s, inv));
        *reinterpret_cast<uint2*>(&qcodes[wave][sub * 8]) = w;
        if (sub == 0) qscale[wave] = s;
      }
    }
    __syncthreads();
    int32_t qw[D / 4];
    float qs = 1.0f;
    if (active) {
#pragma unroll
      for (int w = 0; w < D / 4; ++w) qw[w] = reinterpret_cast<const int32_t*>(qcodes[wave])[w];
      qs = qscale[wave];
    }
    // anchor: the largest score over the anchor region (keys read from global)
    float anchor = -__builtin_inff();
    if (active) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int k = u == 0 ? lane : loc0 + 64 * (u - 1) + lane;
        if (k < nvis && (u == 0 || k >= kKBlock)) {
          const float sc = key_score<D>(qw, a.k_i8 + (krow0 + k) * D, qs, kscale[k / kKBlock]);
          anchor = __builtin_fmaxf(anchor, sc);
        }
      }
      anchor = wave_max(anchor);
    }
    const float thr = anchor - a.theta;
    const int room = a.max_keys - nregion;  // capacity left for keys outside the region
    int32_t* out = a.key_idx + row * a.max_keys;
    int written = 0, others = 0;
    for (int c0 = 0; c0 < nvis; c0 += kChunk) {
      const int cn = min(kChunk, nvis - c0);
      __syncthreads();
      {
        constexpr int CPR = D / 16;
        const int8_t* ksrc = a.k_i8 + (krow0 + c0) * D;
        for (int c = threadIdx.x; c < cn * CPR; c += kThreads) {
          const int kk = c / CPR;
          const int part = c % CPR;
          *reinterpret_cast<int4*>(&kcodes[kk * KSTR + part * 16]) =
              *reinterpret_cast<const int4*>(ksrc + (size_t)kk * D + part * 16);
        }
      }
      __syncthreads();
      if (!active) continue;
#pragma unroll
      for (int u = 0; u < kChunk / 64; ++u) {
        const int k = c0 + 64 * u + lane;
        const bool valid = 64 * u + lane < cn;
        bool keep = false, reg = false;
        if (valid) {
          reg = in_region(k);
          const float sc = key_score<D>(qw, &kcodes[(64 * u + lane) * KSTR], qs, kscale[k / kKBlock]);
          keep = reg || sc >= thr;
        }
        // others past the room are dropped, lowest indices first kept
        const bool other = keep && !reg;
        const uint64_t ob = __ballot(other);
        const int orank = others + __popcll(ob & lt_mask);
        others += __popcll(ob);
        const bool write = reg || (other && orank < room);
        const uint64_t wb = __ballot(valid && write);
        if (valid && write) out[written + __popcll(wb & lt_mask)] = k;
        written += __popcll(wb);
      }
    }
    if (!active) continue;
    for (int pos = written + lane; pos < a.max_keys; pos += 64) out[pos] = -1;
    if (lane == 0) a.key_cnt[row] = written;
  }
}

}  // namespace

hipError_t launch_stripe_select(const Shape& s, const float* q_pool, const int8_t* k_i8,
                                const float* k_scale, float theta, int max_keys,
                                int32_t* key_idx, int32_t* key_cnt, hipStream_t stream) {
  StripeArgs a;
  a.q_pool = q_pool;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.key_idx = key_idx;
  a.key_cnt = key_cnt;
  a.theta = theta;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.group = s.Hq / s.Hkv;
  a.N = s.N;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.causal = s.causal;
  a.max_keys = max_keys;
  const dim3 grid(s.B * s.Hkv * s.nqb());
  if (s.d == 128) hipLaunchKernelGGL(stripe_select_kernel<128>, grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(stripe_select_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qattn
