// Anchor-based stripe selection: per (b, hq, query block), the key positions
// whose score comes within a threshold of the anchor.
//
// A workgroup of 8 waves takes 32 query vectors of one (b, kv head): the
// mean queries of consecutive (query block, query head) pairs of the head
// group, the query block outer. It INT8-quantizes them (the pooled-mask
// rule) and finds each one's anchor over its anchor region (the first 64 keys
// and its block's own 128 positions) with v_dot4 straight from global memory.
// Then it streams the keys once for all 32: each wave takes every eighth
// group of 32 keys and forms the 32 x 32 code products with
// v_mfma_i32_32x32x32_i8 (key rows as A, the query codes as B), so a key row
// read from memory serves 32 query vectors; the key rows are loaded two steps
// ahead. The score is the exact int32 product with two fp32 roundings, as in
// the pooled mask. Per group the kept keys of each query vector become two
// 32-bit masks (anchor-region keys, other kept keys); the waves swap their
// masks' counts through LDS, and the counts of the waves before plus
// popcounts within the wave's own masks give every kept key its place in the
// ascending list. Past the capacity only anchor-region keys are written.
#include "device_util.h"
#include "qattn_internal.h"

#pragma clang fp contract(off)

namespace qattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 32;                    // query vectors per workgroup (the product's N)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

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
  constexpr int KS = D / 32;  // 32-deep k-steps of the product
  __shared__ __attribute__((aligned(16))) int8_t qcodes[kCols][D];
  __shared__ float qscale[kCols];
  __shared__ float thr_s[kCols];
  // per step, wave and column: anchor-region keys << 16 | other kept keys
  __shared__ uint32_t mcnt[2][kWaves][kCols];
  __shared__ int cnt_s[kCols];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int nvec = a.group * a.nqb;  // query vectors of one (b, kv head)
  const int units = (nvec + kCols - 1) / kCols;
  const int slot = blockIdx.x % (a.B * a.Hkv);
  const int rank = blockIdx.x / (a.B * a.Hkv);
  const int u = a.causal ? units - 1 - rank : rank;  // longest key ranges first
  const int b = slot / a.Hkv;
  const int hk = slot % a.Hkv;
  const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.N;
  const float* kscale = a.k_scale + ((size_t)b * a.Hkv + hk) * a.nkb;
  const int ncols = min(kCols, nvec - kCols * u);  // >= 1
  // column c: query block (32u + c) / group of query head hk*group + (32u + c) % group
  auto col_block = [&](int c) { return (kCols * u + c) / a.group; };
  auto col_row = [&](int c) -> size_t {
    const int f = kCols * u + c;
    return ((size_t)b * a.Hq + hk * a.group + f % a.group) * a.nqb + f / a.group;
  };
  auto col_nvis = [&](int c) -> int {
    if (c >= ncols) return 0;
    return a.causal ? min(a.N, kQBlock * col_block(c) + kQBlock) : a.N;
  };

  // the mean queries' INT8 codes: 16 threads per column, 8 channels each
  if (threadIdx.x < 16 * kCols) {
    constexpr int LPV = D / 8;
    const int c = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;
    const bool has = c < ncols && sub < LPV;
    const float* src = a.q_pool + col_row(c < ncols ? c : 0) * D + sub * 8;
    float v[8];
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = has ? src[e] : 0.0f;
      am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o, 64));
    const float sc = quant_scale(am);
    const float inv = 1.0f / sc;
    if (sub < LPV) {
      uint2 w;
      w.x = pack4_i8(quant_code(v[0], sc, inv), quant_code(v[1], sc, inv),
                     quant_code(v[2], sc, inv), quant_code(v[3], sc, inv));
      w.y = pack4_i8(quant_code(v[4], sc, inv), quant_code(v[5], sc, inv),
                     quant_code(v[6], sc, inv), quant_code(v[7], sc, inv));
      *reinterpret_cast<uint2*>(&qcodes[c][sub * 8]) = w;
    }
    if (sub == 0) qscale[c] = sc;
  }
  __syncthreads();

  // anchors: wave w takes columns w, w + 8, ...; lanes score keys (every lane
  // scores a valid row, key 0 in place of an unused one, so that the three
  // rows' loads are all in flight together)
  for (int c = wave; c < kCols; c += kWaves) {
    const int nv = col_nvis(c);
    float anchor = -__builtin_inff();
    if (nv > 0) {
      int32_t qw[D / 4];
#pragma unroll
      for (int w = 0; w < D / 4; ++w) qw[w] = reinterpret_cast<const int32_t*>(qcodes[c])[w];
      const float qs = qscale[c];
      const int loc0 = kQBlock * col_block(c);
#pragma unroll
      for (int u3 = 0; u3 < 3; ++u3) {
        const int k = u3 == 0 ? lane : loc0 + 64 * (u3 - 1) + lane;
        const bool use = k < nv && (u3 == 0 || k >= kKBlock);
        const int kk = use ? k : 0;
        const float sc = key_score<D>(qw, a.k_i8 + (krow0 + kk) * D, qs, kscale[kk / kKBlock]);
        anchor = __builtin_fmaxf(anchor, use ? sc : -__builtin_inff());
      }
      anchor = wave_max(anchor);
    }
    if (lane == 0) thr_s[c] = nv > 0 ? anchor - a.theta : __builtin_inff();
  }
  __syncthreads();

  // this lane's column (both lane halves keep the same running counts)
  const int c = l32;
  const int nv = col_nvis(c);
  const int loc0 = kQBlock * col_block(c);
  const float thr = thr_s[c];
  const float qs = qscale[c];
  const int nreg = nv > 0 ? min(kKBlock, nv) + max(0, min(nv, loc0 + kQBlock) - max(loc0, kKBlock)) : 0;
  const int room = a.max_keys - nreg;  // capacity left for keys outside the anchor region
  v4i qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const v4i*>(&qcodes[c][32 * ks + 16 * h]);
  int32_t* out = a.key_idx + col_row(nv > 0 ? c : 0) * a.max_keys;
  // the workgroup's key range (the last column has the longest) and the span
  // of its anchor windows; groups outside [0, 64), outside every window and
  // below every column's visible range need no region or visibility test
  const int nv_max = col_nvis(ncols - 1);
  const int nv_min = col_nvis(0);
  const int win_lo = kQBlock * col_block(0);
  const int win_hi = kQBlock * col_block(ncols - 1) + kQBlock;

  const int ngroups = nv_max / 32;
  const int iters = (ngroups + kWaves - 1) / kWaves;

  // group g's key rows (A operand) and, issued right behind them, its block
  // scale (a vector load: waiting for it is waiting for the same group's rows)
  auto load_k = [&](int g, v4i (&kf)[KS], float& ksc) {
    const int8_t* src = a.k_i8 + (krow0 + 32 * g + l32) * D + 16 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const v4i*>(src + 32 * ks);
    ksc = kscale[(32 * g) / kKBlock];
  };
  // element r of the product holds key row 8*(r/4) + 4*h + r%4 of the group
  auto spread = [&](uint32_t m16) {
    uint32_t m = 0;
#pragma unroll
    for (int n = 0; n < 4; ++n) m |= ((m16 >> (4 * n)) & 0xFu) << (8 * n + 4 * h);
    return m;
  };
  auto both_halves = [](uint32_t m) {
    const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return m | (uint32_t)sw[0] | (uint32_t)sw[1];
  };
  // workgroup barrier that waits for LDS traffic only: the key loads in
  // flight (two steps ahead) and the list stores need no wait here
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  int R = 0, O = 0;  // anchor-region keys and other kept keys so far
  // step it: this wave's group it*8 + wave, whose key rows and scale were
  // loaded two steps earlier; kf then takes the group two ahead (the last
  // group again past the end: a load on every path, so that the loaded
  // registers need no copy, and no wait, at a join)
  auto step = [&](int it, v4i (&kf)[KS], float& ksc_ref) {
    const int g = it * kWaves + wave;
    const int key0 = 32 * g;
    uint32_t reg16 = 0, oth16 = 0;
    bool plain = true;  // no anchor-region key and no visibility test in the group
    if (g < ngroups) {  // wave-uniform
      v16i acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[ks], qf[ks], acc, 0, 0, 0);
      const float ksc = ksc_ref;
      plain = key0 >= kKBlock && (key0 + 32 <= win_lo || key0 >= win_hi) &&
              key0 + 32 <= nv_min;
      if (plain) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sc = ((float)(int)acc[r] * qs) * ksc;
          oth16 |= (sc >= thr ? 1u : 0u) << r;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float sc = ((float)(int)acc[r] * qs) * ksc;
          const bool vis = key < nv;
          const bool reg = key < kKBlock || (key >= loc0 && key < loc0 + kQBlock);
          reg16 |= (vis && reg ? 1u : 0u) << r;
          oth16 |= (vis && !reg && sc >= thr ? 1u : 0u) << r;
        }
      }
    }
    load_k(min(g + 2 * kWaves, ngroups - 1), kf, ksc_ref);
    const uint32_t reg32 = plain ? 0u : both_halves(spread(reg16));  // (uniform)
    const uint32_t oth32 = both_halves(spread(oth16));
    const int buf = it & 1;
    // (at most 32 keys per group and wave: the packed sums cannot carry)
    if (h == 0)
      mcnt[buf][wave][l32] = ((uint32_t)__builtin_popcount(reg32) << 16) |
                             (uint32_t)__builtin_popcount(oth32);
    barrier();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t v = mcnt[buf][w][l32];
      pre += w < wave ? v : 0u;
      tot += v;
    }
    const int rpre = (int)(pre >> 16), opre = (int)(pre & 0xFFFFu);
    const int rtot = (int)(tot >> 16), otot = (int)(tot & 0xFFFFu);
    uint32_t mine = reg16 | oth16;
    while (mine != 0u) {
      const int r = __builtin_ctz(mine);
      mine &= mine - 1u;
      const int kr = 8 * (r >> 2) + 4 * h + (r & 3);
      const uint32_t below = (1u << kr) - 1u;
      const int rb = R + rpre + __builtin_popcount(reg32 & below);
      const int ob = O + opre + __builtin_popcount(oth32 & below);
      if ((reg16 >> r) & 1u) out[rb + min(ob, room)] = key0 + kr;
      else if (ob < room) out[rb + ob] = key0 + kr;
    }
    R += rtot;
    O += otot;
  };
  v4i kfa[KS], kfb[KS];
  float ksa, ksb;
  load_k(min(wave, ngroups - 1), kfa, ksa);
  load_k(min(wave + kWaves, ngroups - 1), kfb, ksb);
  for (int it = 0; it < iters; it += 2) {
    step(it, kfa, ksa);
    if (it + 1 < iters) step(it + 1, kfb, ksb);
  }
  if (wave == 0 && h == 0) {
    const int total = R + min(O, room);
    cnt_s[c] = nv > 0 ? total : -1;
    if (nv > 0) a.key_cnt[col_row(c)] = total;
  }
  __syncthreads();
  for (int cc = 0; cc < ncols; ++cc) {
    int32_t* o2 = a.key_idx + col_row(cc) * a.max_keys;
    for (int pos = cnt_s[cc] + threadIdx.x; pos < a.max_keys; pos += kThreads) o2[pos] = -1;
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
  const int units = (a.group * a.nqb + kCols - 1) / kCols;
  const dim3 grid(s.B * s.Hkv * units);
  if (s.d == 128) hipLaunchKernelGGL(stripe_select_kernel<128>, grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(stripe_select_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qattn
