// Element-level 4-bit block estimator (the SALE-style mask).
//
// Three launches on the caller's stream:
//   1. mxfp4_quant -- the raw Q and the smoothed K (fl32(K) - k_mean) to OCP
//      MX FP4: E2M1 codes, two per byte (even channel in the low nibble), and
//      one E8M0 exponent byte per 32 channels. Four lanes share a group of 32
//      channels (8 each); the shared exponent is floor(log2 amax) - 2, read
//      from amax's exponent field; codes round to nearest-even on the E2M1
//      grid by a sum of threshold tests (ties resolved by which side of each
//      threshold is inclusive) and saturate at 6.
//   2. lowbit_score -- one 4-wave workgroup per (b, kv head, query block),
//      one query head of the group per wave and round. A wave holds the MX
//      fragments of its 128 query rows and, per causally valid key block,
//      scores all 128 x 64 pairs with v_mfma_scale_f32_32x32x64_f8f6f4 (FP4
//      operands, the E8M0 scales applied per 32 channels by the matrix core),
//      masks the invisible pairs and reduces them to the block's largest
//      estimate. The four waves of a workgroup read the same key block, so
//      its second and later reads hit the CU's cache.
//   3. the pooled mask's selection (forced + top fraction, ties to the lower
//      block index) on these scores.
#include <type_traits>

#include "../../include/qattn.h"
#include "device_util.h"
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kMx = 32;  // channels per E8M0 scale

struct LowbitLayout {
  uint8_t* q4;  // [B*Hq*N][d/2]
  uint8_t* qe;  // [B*Hq*N][d/32]
  uint8_t* k4;  // [B*Hkv*N][d/2]
  uint8_t* ke;  // [B*Hkv*N][d/32]
  float* scores;  // [B*Hq*nqb][nkb]
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LowbitLayout lowbit_layout(void* ws, const Shape& s, float* scores) {
  const size_t nq = (size_t)s.B * s.Hq * s.N;
  const size_t nk = (size_t)s.B * s.Hkv * s.N;
  uint8_t* p = static_cast<uint8_t*>(ws);
  LowbitLayout L;
  L.q4 = p;
  p += align256(nq * s.d / 2);
  L.qe = p;
  p += align256(nq * s.d / kMx);
  L.k4 = p;
  p += align256(nk * s.d / 2);
  L.ke = p;
  p += align256(nk * s.d / kMx);
  L.scores = scores != nullptr ? scores : reinterpret_cast<float*>(p);
  return L;
}

// E2M1 magnitude code of a >= 0 (already divided by the shared scale):
// nearest grid point of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
// saturating at 6
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const float* __restrict__ k_mean,
                                                          LowbitLayout L, long long nq_rows,
                                                          long long nk_rows, int N) {
  constexpr int LPR = D / 8;  // lanes per row, 8 channels each
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  const bool ok = row < nq_rows + nk_rows;
  const bool isq = row < nq_rows;
  const long long r = isq ? row : row - nq_rows;
  float x[8];
  if (ok) {
    const uint16_t* src = (isq ? q : k) + r * D + sub * 8;
    load8_f32<BF16>(src, x);
    if (!isq) {
      const float* m = k_mean + (r / N) * D + sub * 8;  // per (b, kv head)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] - m[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.0f;
  }
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(x[e]));
  am = __builtin_fmaxf(am, __shfl_xor(am, 1, 64));
  am = __builtin_fmaxf(am, __shfl_xor(am, 2, 64));
  if (!ok) return;
  // shared exponent floor(log2 amax) - 2, at least -127 (zero or tiny groups)
  const int ef = (int)((__float_as_uint(am) >> 23) & 0xffu);
  const int E = ef == 0 ? -127 : max(ef - 129, -127);
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = __builtin_ldexpf(__builtin_fabsf(x[e]), -E);
    const uint32_t nib = e2m1_code(y) | (x[e] < 0.0f ? 8u : 0u);
    packed |= nib << (4 * e);
  }
  *reinterpret_cast<uint32_t*>((isq ? L.q4 : L.k4) + r * (D / 2) + sub * 4) = packed;
  if ((sub & 3) == 0) (isq ? L.qe : L.ke)[r * (D / kMx) + sub / 4] = (uint8_t)(E + 127);
}

// Max over the 64 lanes without LDS round trips (a shuffle chain waits for
// each of its six LDS permutes): DPP butterflies within each row of 16 lanes
// (xor 1 and xor 2 by quad permutes, then the half-row and row mirrors), then
// the row broadcasts of lanes 15 and 31 fold the four rows upward. Lane 63
// ends with the maximum over all lanes.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
  const int x = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK,
                                            0xF, false);
  return __builtin_fmaxf(v, __int_as_float(x));
}
__device__ __forceinline__ float wave_max_to_lane63(float v) {
  v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max<0x140, 0xF>(v);  // row_mirror: every lane holds its row's max
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

struct ScoreArgs {
  LowbitLayout L;
  int B, Hq, Hkv, group, N, nqb, nkb, causal;
};

template <int D>
__global__ __launch_bounds__(256) void lowbit_score_kernel(ScoreArgs a) {
  constexpr int KS = D / 64;  // 64-channel k-steps of the FP4 product
  constexpr int RB = 4;       // 32-row blocks of a 128-row query block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  // longest causal rows first
  const int slot = blockIdx.x % (a.B * a.Hkv);
  const int rank = blockIdx.x / (a.B * a.Hkv);
  const int i = a.causal ? a.nqb - 1 - rank : rank;
  const int b = slot / a.Hkv;
  const int hk = slot % a.Hkv;
  const int nvalid = a.causal ? min(a.nkb, (kQBlock * i + kQBlock - 1) / kKBlock + 1) : a.nkb;
  const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.N;
  const int rounds = (a.group + 3) / 4;
  for (int round = 0; round < rounds; ++round) {
    const int g = round * 4 + wave;
    if (g >= a.group) break;  // wave-uniform
    const int hq = hk * a.group + g;
    const size_t bhq = (size_t)b * a.Hq + hq;
    // B operand: query row 128 i + 32 rb + l32, channels 64 ks + 32 h + [0, 32)
    v8i qf[RB][KS];
    int qs[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const size_t qr = bhq * a.N + kQBlock * i + 32 * rb + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = *reinterpret_cast<const uint4*>(a.L.q4 + qr * (D / 2) + 32 * ks + 16 * h);
        qf[rb][ks] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        qs[rb][ks] = a.L.qe[qr * (D / kMx) + 2 * ks + h];
      }
    }
    float* out = a.L.scores + (bhq * a.nqb + i) * a.nkb;
    // Key block j's A-operand fragments (key 64 j + 32 kb + l32, channels
    // 64 ks + 32 h + [0, 32)) and their E8M0 scales; the loop loads block
    // j + 1 while it scores block j.
    struct KFrag {
      v8i f[2][KS];
      int e[2][KS];
    };
    auto load_kblock = [&](int j, KFrag& kf) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const size_t kr = krow0 + kKBlock * j + 32 * kb + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 w = *reinterpret_cast<const uint4*>(a.L.k4 + kr * (D / 2) + 32 * ks + 16 * h);
          kf.f[kb][ks] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
          kf.e[kb][ks] = a.L.ke[kr * (D / kMx) + 2 * ks + h];
        }
      }
    };
    // Per key block: the masked (diagonal) blocks take the element test, the
    // others none; four running maxima per lane keep the max chains short.
    auto score_block = [&](int j, const KFrag& kf, auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
      float best[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // two 32-row blocks at a time, their k-steps interleaved, so that no
        // matrix instruction waits for the one just before it
#pragma unroll
        for (int rp = 0; rp < RB; rp += 2) {
          v16f s[2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[u][r] = 0.0f;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int u = 0; u < 2; ++u)
              s[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  kf.f[kb][ks], qf[rp + u][ks], s[u], 4, 4, 0, kf.e[kb][ks], 0, qs[rp + u][ks]);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // element r: key 64 j + 32 kb + 8 (r/4) + 4 h + r%4, query 128 i + 32 (rp+u) + l32
            const int lim = (32 * (rp + u) + l32) + kQBlock * i - (kKBlock * j + 32 * kb + 4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float v = s[u][r];
              if constexpr (DIAG) {
                const int off = 8 * (r >> 2) + (r & 3);
                v = off > lim ? -__builtin_inff() : v;
              }
              best[r & 3] = __builtin_fmaxf(best[r & 3], v);
            }
          }
        }
      }
      return __builtin_fmaxf(__builtin_fmaxf(best[0], best[1]), __builtin_fmaxf(best[2], best[3]));
    };
    // the last key blocks of a causal query block need the element test
    const int nplain = a.causal ? min(nvalid, (kQBlock * i + 1) / kKBlock) : nvalid;
    auto finish = [&](int j, const KFrag& kf) {
      float best = j < nplain ? score_block(j, kf, std::integral_constant<bool, false>{})
                              : score_block(j, kf, std::integral_constant<bool, true>{});
      best = wave_max_to_lane63(best);
      if (lane == 63) out[j] = best;
    };
    // The prefetches are unconditional (clamped to the last block, whose
    // extra load is harmless): with a fixed number of loads in flight the
    // compiler waits only for the older block's loads, not for every load.
    KFrag ka, kb2;
    load_kblock(0, ka);
    for (int j = 0; j < nvalid; j += 2) {
      load_kblock(min(j + 1, nvalid - 1), kb2);
      finish(j, ka);
      load_kblock(min(j + 2, nvalid - 1), ka);
      if (j + 1 < nvalid) finish(j + 1, kb2);
    }
  }
}

}  // namespace

size_t lowbit_workspace_bytes(const Shape& s, bool with_scores) {
  const size_t nq = (size_t)s.B * s.Hq * s.N;
  const size_t nk = (size_t)s.B * s.Hkv * s.N;
  size_t n = align256(nq * s.d / 2) + align256(nq * s.d / kMx) + align256(nk * s.d / 2) +
             align256(nk * s.d / kMx);
  if (with_scores) n += (size_t)s.B * s.Hq * s.nqb() * s.nkb() * sizeof(float);
  return n;
}

namespace {

void launch_quant(const Shape& s, const void* q, const void* k, const float* k_mean,
                  const LowbitLayout& L, hipStream_t stream) {
  const long long nq_rows = (long long)s.B * s.Hq * s.N;
  const long long nk_rows = (long long)s.B * s.Hkv * s.N;
  const int rows_per_block = 256 / (s.d / 8);
  const long long qgrid = (nq_rows + nk_rows + rows_per_block - 1) / rows_per_block;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  if (s.d == 128) {
    if (s.bf16)
      hipLaunchKernelGGL((mxfp4_quant_kernel<128, true>), dim3((unsigned)qgrid), dim3(256), 0,
                         stream, q16, k16, k_mean, L, nq_rows, nk_rows, s.N);
    else
      hipLaunchKernelGGL((mxfp4_quant_kernel<128, false>), dim3((unsigned)qgrid), dim3(256), 0,
                         stream, q16, k16, k_mean, L, nq_rows, nk_rows, s.N);
  } else {
    if (s.bf16)
      hipLaunchKernelGGL((mxfp4_quant_kernel<64, true>), dim3((unsigned)qgrid), dim3(256), 0,
                         stream, q16, k16, k_mean, L, nq_rows, nk_rows, s.N);
    else
      hipLaunchKernelGGL((mxfp4_quant_kernel<64, false>), dim3((unsigned)qgrid), dim3(256), 0,
                         stream, q16, k16, k_mean, L, nq_rows, nk_rows, s.N);
  }
}

}  // namespace

Fp4Codes fp4_codes(void* workspace, const Shape& s) {
  const LowbitLayout L = lowbit_layout(workspace, s, nullptr);
  return Fp4Codes{L.q4, L.qe, L.k4, L.ke};
}

hipError_t launch_mxfp4_quant(const Shape& s, const void* q, const void* k, const float* k_mean,
                              void* workspace, hipStream_t stream) {
  launch_quant(s, q, k, k_mean, lowbit_layout(workspace, s, nullptr), stream);
  return hipGetLastError();
}

hipError_t launch_lowbit_mask(const Shape& s, const void* q, const void* k, const float* k_mean,
                              int keep_num, int keep_den, int max_keep, int32_t* kv_idx,
                              int32_t* kv_cnt, float* scores, void* workspace,
                              hipStream_t stream) {
  const LowbitLayout L = lowbit_layout(workspace, s, scores);
  launch_quant(s, q, k, k_mean, L, stream);
  ScoreArgs sa;
  sa.L = L;
  sa.B = s.B;
  sa.Hq = s.Hq;
  sa.Hkv = s.Hkv;
  sa.group = s.Hq / s.Hkv;
  sa.N = s.N;
  sa.nqb = s.nqb();
  sa.nkb = s.nkb();
  sa.causal = s.causal;
  const dim3 sgrid(s.B * s.Hkv * s.nqb());
  if (s.d == 128) hipLaunchKernelGGL(lowbit_score_kernel<128>, sgrid, dim3(256), 0, stream, sa);
  else hipLaunchKernelGGL(lowbit_score_kernel<64>, sgrid, dim3(256), 0, stream, sa);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select_scores(s, L.scores, keep_num, keep_den, max_keep, kv_idx, kv_cnt, stream);
}

}  // namespace qattn
