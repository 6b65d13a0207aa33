// Vertical and slash pattern prediction on top of a block plan.
//
// The SALE explainer (aibr.jp/archives/118208), sections 1 and 3: besides the
// element-level estimates, the method predicts vertical lines (key positions
// every query needs) and slash lines (a fixed query-key distance) from the
// attention map's tendencies. Reading: every query block votes with the
// non-forced blocks of its kept set (the valid entries of its list, once
// each; forced are block 0 and the diagonal blocks 2i, 2i+1) for their key
// block j (vertical) and for their offset o = 2i - j (slash). The n_vertical
// key blocks and n_slash offsets with the most votes, at least two, ties to
// the lower index, are the head's lines; every query block then keeps its own
// set plus the valid blocks on those lines, in ascending order.
//
// Two launches:
//  1. pattern_vote_kernel, one 1024-thread workgroup per (b, hq): each of
//     its 16 waves takes every sixteenth query block, marks the block's
//     valid entries in its own LDS bit set and adds one vote per marked,
//     non-forced block to the head's counters in LDS; then the lines, one
//     workgroup argmax per line over packed keys (votes << 16 |
//     (65535 - index)), written to `lines`.
//  2. pattern_extend_kernel, one wave per (b, hq, query block): the bit set
//     of the block's valid entries and the valid blocks on its head's lines,
//     compacted in ascending order with popcounts and a wave prefix sum.
#include <limits.h>

#include "../../include/qattn.h"
#include "qattn_internal.h"

namespace qattn {
namespace {

constexpr int kMaxNkb = 2048;           // key blocks (N <= 131072)
constexpr int kWords = kMaxNkb / 32;    // bit-set dwords, one per lane
constexpr int kThreads = 256;           // extend: one wave per query block
constexpr int kWaves = kThreads / 64;
constexpr int kVoteThreads = 1024;      // votes: 16 waves share a head's query blocks
constexpr int kVoteWaves = kVoteThreads / 64;

struct PatArgs {
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  int32_t* kv_idx_out;
  int32_t* kv_cnt_out;
  int32_t* lines;  // [B*Hq][n_v + n_s]
  int nqb, nkb, max_keep, max_keep_out, n_v, n_s, rows;
  bool causal;
};

__device__ __forceinline__ bool valid_block(int j, int i, int nkb, bool causal) {
  return j >= 0 && j < nkb && (!causal || j <= 2 * i + 1);
}

// order LDS traffic of the lanes of one wave (plain stores before atomics)
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The valid entries of query block i's list as a bit set: lane l owns blocks
// [32 l, 32 l + 32) in bits[l]. Returns this lane's word.
__device__ __forceinline__ uint32_t mark_list(const PatArgs& a, const int32_t* row, int cnt, int i,
                                              uint32_t* bits, int lane) {
  bits[lane] = 0u;
  wave_lds_fence();
  const int n = min(max(cnt, 0), a.max_keep);
  for (int e = lane; e < n; e += 64) {
    const int j = row[e];
    if (valid_block(j, i, a.nkb, a.causal)) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  wave_lds_fence();
  return bits[lane];
}

// forced blocks of query block i within lane's word
__device__ __forceinline__ uint32_t forced_word(int i, int lane, int nkb, bool causal) {
  uint32_t f = 0u;
  const int js[3] = {0, 2 * i, 2 * i + 1};
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const int j = js[x];
    if (valid_block(j, i, nkb, causal) && (j >> 5) == lane) f |= 1u << (j & 31);
  }
  return f;
}

__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}

__global__ __launch_bounds__(kVoteThreads) void pattern_vote_kernel(PatArgs a) {
  __shared__ int vert[kMaxNkb];
  __shared__ int slash[2 * kMaxNkb];
  __shared__ uint32_t bits[kVoteWaves][kWords];
  __shared__ unsigned red[kVoteWaves];
  const int head = blockIdx.x;  // b * Hq + hq
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslash = 2 * a.nkb - 1;
  for (int x = tid; x < a.nkb; x += kVoteThreads) vert[x] = 0;
  for (int x = tid; x < nslash; x += kVoteThreads) slash[x] = 0;
  __syncthreads();
  for (int i = wave; i < a.nqb; i += kVoteWaves) {
    const size_t r = (size_t)head * a.nqb + i;
    uint32_t w = mark_list(a, a.kv_idx + r * a.max_keep, a.kv_cnt[r], i, bits[wave], lane);
    w &= ~forced_word(i, lane, a.nkb, a.causal);
    while (w != 0u) {
      const int p = __builtin_ctz(w);
      w &= w - 1u;
      const int j = 32 * lane + p;
      atomicAdd(&vert[j], 1);
      atomicAdd(&slash[2 * i - j + a.nkb - 1], 1);
    }
  }
  __syncthreads();
  // the lines: repeated argmax over (votes, lower index), at least two votes
  int32_t* out = a.lines + (size_t)head * (a.n_v + a.n_s);
  for (int kind = 0; kind < 2; ++kind) {
    int* cnt = kind == 0 ? vert : slash;
    const int n = kind == 0 ? a.nkb : nslash;
    const int want = kind == 0 ? a.n_v : a.n_s;
    for (int r = 0; r < want; ++r) {
      unsigned best = 0u;
      for (int x = tid; x < n; x += kVoteThreads) {
        const int v = cnt[x];
        if (v >= 2) best = max(best, ((unsigned)v << 16) | (unsigned)(65535 - x));
      }
      best = wave_max_u32(best);
      if (lane == 0) red[wave] = best;
      __syncthreads();
      best = 0u;
#pragma unroll
      for (int w = 0; w < kVoteWaves; ++w) best = max(best, red[w]);
      const int x = 65535 - (int)(best & 0xffffu);
      if (tid == 0) {
        if (kind == 0) out[r] = best != 0u ? x : -1;
        else out[a.n_v + r] = best != 0u ? x - (a.nkb - 1) : INT_MIN;
        if (best != 0u) cnt[x] = 0;
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kThreads) void pattern_extend_kernel(PatArgs a) {
  __shared__ uint32_t bits[kWaves][kWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * kWaves + wave;  // (b * Hq + hq) * nqb + i
  if (r >= a.rows) return;
  const int head = r / a.nqb, i = r % a.nqb;
  const int32_t* lines = a.lines + (size_t)head * (a.n_v + a.n_s);
  mark_list(a, a.kv_idx + (size_t)r * a.max_keep, a.kv_cnt[r], i, bits[wave], lane);
  if (lane < a.n_v) {
    const int j = lines[lane];
    if (valid_block(j, i, a.nkb, a.causal)) atomicOr(&bits[wave][j >> 5], 1u << (j & 31));
  }
  if (lane < a.n_s) {
    const int o = lines[a.n_v + lane];
    if (o != INT_MIN) {
      const int j = 2 * i - o;
      if (valid_block(j, i, a.nkb, a.causal)) atomicOr(&bits[wave][j >> 5], 1u << (j & 31));
    }
  }
  wave_lds_fence();
  uint32_t w = bits[wave][lane];
  const int pc = __builtin_popcount(w);
  // exclusive prefix of the popcounts over the lanes
  int incl = pc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  int pos = incl - pc;
  int32_t* dst = a.kv_idx_out + (size_t)r * a.max_keep_out;
  while (w != 0u) {
    const int p = __builtin_ctz(w);
    w &= w - 1u;
    if (pos < a.max_keep_out) dst[pos] = 32 * lane + p;
    ++pos;
  }
  for (int e = total + lane; e < a.max_keep_out; e += 64) dst[e] = -1;
  if (lane == 0) a.kv_cnt_out[r] = min(total, a.max_keep_out);
}

}  // namespace

int pattern_max_nkb() { return kMaxNkb; }

hipError_t launch_patterns(const Shape& s, const int32_t* kv_idx, const int32_t* kv_cnt,
                           int max_keep, int n_vertical, int n_slash, int32_t* kv_idx_out,
                           int32_t* kv_cnt_out, int max_keep_out, int32_t* lines,
                           hipStream_t stream) {
  PatArgs a;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.kv_idx_out = kv_idx_out;
  a.kv_cnt_out = kv_cnt_out;
  a.lines = lines;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.max_keep = max_keep;
  a.max_keep_out = max_keep_out;
  a.n_v = n_vertical;
  a.n_s = n_slash;
  a.rows = s.B * s.Hq * a.nqb;
  a.causal = s.causal != 0;
  hipLaunchKernelGGL(pattern_vote_kernel, dim3(s.B * s.Hq), dim3(kVoteThreads), 0, stream, a);
  hipLaunchKernelGGL(pattern_extend_kernel, dim3((a.rows + kWaves - 1) / kWaves), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace qattn
