// Block mask: per (b, hq, query block), the kept key blocks.
//
// Two launches on the caller's stream:
//   1. pool_quant -- INT8-quantize every pooled query and key vector on its
//      own (codes + fp32 scale into the workspace); one 16-lane (d = 128) or
//      8-lane (d = 64) group per vector.
//   2. select     -- one workgroup per (b, hk, query block); wave w takes query
//      heads w, w+4, ... of the group. Per chunk of 256 key blocks the
//      workgroup stages the key codes in LDS; lane l of a wave scores key
//      blocks l, l+64, ... with v_dot4 (exact int32) and two fp32 roundings.
//      A radix select over the order-preserving integer image of the scores
//      (most significant bit first, stopping once the candidates sharing the
//      prefix are exactly the ones still wanted) finds the k-th largest
//      candidate (ties at the threshold go to the lower block index);
//      ballot/popcount prefix sums write forced and selected blocks in
//      ascending order and pad with -1.
#include "device_util.h"
#include "qattn_internal.h"

#pragma clang fp contract(off)

namespace qattn {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kJChunk = 256;

struct MaskLayout {
  int8_t* qc;   // [B*Hq*nqb][d]
  int8_t* kc;   // [B*Hkv*nkb][d]
  float* qs;    // [B*Hq*nqb]
  float* ks;    // [B*Hkv*nkb]
};

__host__ __device__ inline MaskLayout mask_layout(void* ws, const Shape& s) {
  const size_t nq = (size_t)s.B * s.Hq * s.nqb();
  const size_t nk = (size_t)s.B * s.Hkv * s.nkb();
  int8_t* base = static_cast<int8_t*>(ws);
  MaskLayout L;
  L.qc = base;
  L.kc = L.qc + nq * s.d;
  L.qs = reinterpret_cast<float*>(L.kc + nk * s.d);
  L.ks = L.qs + nq;
  return L;
}

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_quant_kernel(const float* __restrict__ q_pool,
                                                                  const float* __restrict__ k_pool,
                                                                  MaskLayout L, int nq, int nk) {
  constexpr int LPV = D / 8;                 // lanes per vector
  constexpr int VPB = kPoolThreads / LPV;    // vectors per block
  const int sub = threadIdx.x % LPV;
  const int vec = blockIdx.x * VPB + threadIdx.x / LPV;
  const bool ok = vec < nq + nk;
  const bool isq = vec < nq;
  const int vi = isq ? vec : vec - nq;
  const float* src = ok ? (isq ? q_pool : k_pool) + (size_t)vi * D + sub * 8 : q_pool;
  float v[8];
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = ok ? src[e] : 0.0f;
    am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
  }
#pragma unroll
  for (int o = LPV / 2; o > 0; o >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o, 64));
  if (!ok) return;
  const float s = quant_scale(am);
  const float inv = 1.0f / s;
  uint2 w;
  w.x = pack4_i8(quant_code(v[0], s, inv), quant_code(v[1], s, inv), quant_code(v[2], s, inv),
                 quant_code(v[3], s, inv));
  w.y = pack4_i8(quant_code(v[4], s, inv), quant_code(v[5], s, inv), quant_code(v[6], s, inv),
                 quant_code(v[7], s, inv));
  int8_t* dst = (isq ? L.qc : L.kc) + (size_t)vi * D + sub * 8;
  *reinterpret_cast<uint2*>(dst) = w;
  if (sub == 0) (isq ? L.qs : L.ks)[vi] = s;
}

struct SelArgs {
  MaskLayout L;
  const float* scores;  // [B*Hq*nqb][nkb] when the scores come precomputed
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int B, Hq, Hkv, group, nqb, nkb, causal, keep_num, keep_den, max_keep;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  // -0 and +0 are equal scores: both map to the image of +0
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// FROM_SCORES: the block scores are read from a.scores (the low-bit
// estimator) instead of being formed from the pooled codes.
template <int D, int SLOTS, bool FROM_SCORES>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelArgs a) {
  constexpr int KSTR = D + 16;  // padded LDS row: 16-byte reads of 8 rows hit distinct banks
  __shared__ __attribute__((aligned(16))) int8_t kcodes[FROM_SCORES ? 16 : kJChunk * KSTR];
  __shared__ float kscale[FROM_SCORES ? 1 : kJChunk];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = blockIdx.x % a.nqb;
  const int kvu = blockIdx.x / a.nqb;  // b * Hkv + hk
  const int b = kvu / a.Hkv;
  const int hk = kvu % a.Hkv;
  const int nvalid = a.causal ? min(a.nkb, (kQBlock * i + kQBlock - 1) / kKBlock + 1) : a.nkb;
  const int dlo = (kQBlock * i) / kKBlock;
  const int dhi = (kQBlock * i + kQBlock - 1) / kKBlock;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rounds = (a.group + 3) / 4;

  for (int round = 0; round < rounds; ++round) {
    const int g = round * 4 + wave;
    const bool active = g < a.group;  // wave-uniform
    const int hq = hk * a.group + (active ? g : 0);
    const size_t row = ((size_t)b * a.Hq + hq) * a.nqb + i;
    int32_t qw[D / 4];
    float qs = 1.0f;
    if (active && !FROM_SCORES) {
      const int32_t* qsrc = reinterpret_cast<const int32_t*>(a.L.qc + row * D);
#pragma unroll
      for (int w = 0; w < D / 4; ++w) qw[w] = qsrc[w];
      qs = a.L.qs[row];
    }
    float sc[SLOTS];
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) sc[u] = 0.0f;

    if constexpr (FROM_SCORES) {
      if (active) {
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
          const int j = lane + 64 * u;
          if (j < nvalid) sc[u] = a.scores[row * a.nkb + j];
        }
      }
    }
    for (int j0 = 0; j0 < (FROM_SCORES ? 0 : nvalid); j0 += kJChunk) {
      const int jn = min(kJChunk, nvalid - j0);
      __syncthreads();
      {
        constexpr int CPR = D / 16;  // 16-byte chunks per code row
        const int8_t* ksrc = a.L.kc + ((size_t)kvu * a.nkb + j0) * D;
        for (int c = threadIdx.x; c < jn * CPR; c += kSelThreads) {
          const int jj = c / CPR;
          const int part = c % CPR;
          *reinterpret_cast<int4*>(&kcodes[jj * KSTR + part * 16]) =
              *reinterpret_cast<const int4*>(ksrc + (size_t)jj * D + part * 16);
        }
        for (int jj = threadIdx.x; jj < jn; jj += kSelThreads)
          kscale[jj] = a.L.ks[(size_t)kvu * a.nkb + j0 + jj];
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
          const int j = lane + 64 * u;
          if (j >= j0 && j < j0 + jn) {
            const int4* kr = reinterpret_cast<const int4*>(&kcodes[(j - j0) * KSTR]);
            int dot = 0;
#pragma unroll
            for (int w4 = 0; w4 < D / 16; ++w4) {
              const int4 kk = kr[w4];
              dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 0], kk.x, dot, false);
              dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 1], kk.y, dot, false);
              dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 2], kk.z, dot, false);
              dot = __builtin_amdgcn_sdot4(qw[4 * w4 + 3], kk.w, dot, false);
            }
            const float s1 = (float)dot * qs;
            sc[u] = s1 * kscale[j - j0];
          }
        }
      }
    }
    if (!active) continue;

    uint32_t key[SLOTS];
    bool cand[SLOTS], forced[SLOTS];
    int nforced = 0;
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int j = lane + 64 * u;
      const bool valid = j < nvalid;
      forced[u] = valid && (j == 0 || (j >= dlo && j <= dhi));
      cand[u] = valid && !forced[u];
      key[u] = order_key(sc[u]);
      nforced += __popcll(__ballot(forced[u]));
    }
    const int ncand = nvalid - nforced;
    const long long kwant = ((long long)nvalid * a.keep_num + a.keep_den - 1) / a.keep_den;
    const int ksel = (int)(kwant < ncand ? kwant : ncand);
    // Radix select, most significant bit first: after each bit, `prefix`
    // (under `mask`) is the top bits of the ksel-th largest candidate key,
    // `remaining` how many of the candidates sharing them are still wanted and
    // `group` how many share them. The search stops as soon as the whole group
    // is wanted; a full 32-bit prefix is the key itself (ties: the lower
    // block indices are taken).
    uint32_t thr = 0xffffffffu, mask = 0xffffffffu;
    int need = 0;
    if (ksel > 0) {
      uint32_t prefix = 0;
      int remaining = ksel, group = ncand;
      mask = 0;
      for (int bit = 31; bit >= 0 && group > remaining; --bit) {
        const uint32_t mk = mask | (1u << bit);
        const uint32_t test = prefix | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) cnt += __popcll(__ballot(cand[u] && (key[u] & mk) == test));
        if (cnt >= remaining) {
          prefix = test;
          group = cnt;
        } else {
          remaining -= cnt;
          group -= cnt;
        }
        mask = mk;
      }
      thr = prefix;      // top bits (under mask) of the ksel-th largest candidate
      need = remaining;  // how many candidates with exactly these bits are taken
    }
    int32_t* out = a.kv_idx + row * a.max_keep;
    int eq_before = 0;
    int out_before = 0;
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int j = lane + 64 * u;
      const bool gt = ksel > 0 && cand[u] && (key[u] & mask) > thr;
      const bool eq = ksel > 0 && cand[u] && (key[u] & mask) == thr;
      const uint64_t eqb = __ballot(eq);
      const int eq_rank = eq_before + __popcll(eqb & lt_mask);
      eq_before += __popcll(eqb);
      const bool kept = forced[u] || gt || (eq && eq_rank < need);
      const uint64_t kb = __ballot(kept);
      const int pos = out_before + __popcll(kb & lt_mask);
      out_before += __popcll(kb);
      if (kept) out[pos] = j;
    }
    for (int pos = out_before + lane; pos < a.max_keep; pos += 64) out[pos] = -1;
    if (lane == 0) a.kv_cnt[row] = out_before;
  }
}

template <int D, int SLOTS, bool FROM_SCORES>
void launch_select(const SelArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((select_kernel<D, SLOTS, FROM_SCORES>), dim3(grid), dim3(kSelThreads), 0,
                     stream, a);
}

template <int D, bool FROM_SCORES>
void launch_select_d(const SelArgs& a, int grid, hipStream_t stream) {
  const int slots = (a.nkb + 63) / 64;
  if (slots <= 4) {
    launch_select<D, 4, FROM_SCORES>(a, grid, stream);
  } else if (slots <= 8) {
    launch_select<D, 8, FROM_SCORES>(a, grid, stream);
  } else if (slots <= 16) {
    launch_select<D, 16, FROM_SCORES>(a, grid, stream);
  } else {
    launch_select<D, 32, FROM_SCORES>(a, grid, stream);
  }
}

SelArgs sel_args(const Shape& s, int keep_num, int keep_den, int max_keep, int32_t* kv_idx,
                 int32_t* kv_cnt) {
  SelArgs a;
  a.scores = nullptr;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.group = s.Hq / s.Hkv;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.causal = s.causal;
  a.keep_num = keep_num;
  a.keep_den = keep_den;
  a.max_keep = max_keep;
  return a;
}

}  // namespace

size_t mask_workspace_bytes(const Shape& s) {
  const size_t nq = (size_t)s.B * s.Hq * s.nqb();
  const size_t nk = (size_t)s.B * s.Hkv * s.nkb();
  return (nq + nk) * (size_t)s.d + (nq + nk) * sizeof(float);
}

int mask_max_nkb() { return 2048; }

hipError_t launch_block_mask(const Shape& s, const float* q_pool, const float* k_pool,
                             int keep_num, int keep_den, int max_keep, int32_t* kv_idx,
                             int32_t* kv_cnt, void* workspace, hipStream_t stream) {
  const MaskLayout L = mask_layout(workspace, s);
  const int nq = s.B * s.Hq * s.nqb();
  const int nk = s.B * s.Hkv * s.nkb();
  const int vpb = kPoolThreads / (s.d / 8);
  const int pgrid = (nq + nk + vpb - 1) / vpb;
  if (s.d == 128) {
    hipLaunchKernelGGL(pool_quant_kernel<128>, dim3(pgrid), dim3(kPoolThreads), 0, stream, q_pool,
                       k_pool, L, nq, nk);
  } else {
    hipLaunchKernelGGL(pool_quant_kernel<64>, dim3(pgrid), dim3(kPoolThreads), 0, stream, q_pool,
                       k_pool, L, nq, nk);
  }
  SelArgs a = sel_args(s, keep_num, keep_den, max_keep, kv_idx, kv_cnt);
  a.L = L;
  const int grid = s.B * s.Hkv * a.nqb;
  if (s.d == 128) {
    launch_select_d<128, false>(a, grid, stream);
  } else {
    launch_select_d<64, false>(a, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_select_scores(const Shape& s, const float* scores, int keep_num, int keep_den,
                                int max_keep, int32_t* kv_idx, int32_t* kv_cnt,
                                hipStream_t stream) {
  SelArgs a = sel_args(s, keep_num, keep_den, max_keep, kv_idx, kv_cnt);
  a.L = MaskLayout{};
  a.scores = scores;
  const int grid = s.B * s.Hkv * a.nqb;
  // the score-reading kernel does not depend on d; one instance serves both
  launch_select_d<64, true>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace qattn
