// Quantized attention forward on gfx950 matrix cores.
//
// Work decomposition: one workgroup of two waves per (b, hq, 128-row query
// block); each wave owns 64 query rows (two 32-column MFMA blocks). The grid is
// ordered so that workgroups of one kv head land on one XCD (blockIdx % 8
// selects the XCD) and, for causal masking, the longest rows start first.
//
// Data flow per 64-key tile (all in registers except the K/V staging):
//   S^T[key][q] = K_tile . Q^T           v_mfma_i32_32x32x32_i8, 2x2 blocks
//   online softmax on S^T columns        each lane owns one query column per
//                                        block (lanes l and l+32 hold the two
//                                        halves of its 32 keys)
//   O^T[d][q] += V^T . P^T               v_mfma_f32_32x32x16_{bf16,f16}
// Computing the transposed products makes the INT8 accumulator layout (lane =
// column, registers = rows) exactly the B-operand layout of the 16-bit MFMA, so
// P never leaves registers. K is staged row-major in LDS, V transposed (V^T),
// both with padded rows so the 16- and 8-byte fragment reads are free of bank
// conflicts.
#include "device_util.h"
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <bool BF16>
struct Mma16;

template <>
struct Mma16<true> {
  typedef v8bf op_t;
  typedef __bf16 el_t;
  static __device__ __forceinline__ v16f mma(op_t a, op_t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma16<false> {
  typedef v8h op_t;
  typedef _Float16 el_t;
  static __device__ __forceinline__ v16f mma(op_t a, op_t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

struct FwdArgs {
  const int8_t* q_i8;
  const float* q_scale;
  const int8_t* k_i8;
  const float* k_scale;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  int B, Hq, Hkv, N, group, nqb, nkb, max_keep;
  float c;  // fl32(log2(e) / sqrt(d))
};

constexpr int kThreads = 128;  // two waves
constexpr int kKT = 64;        // keys per tile

template <int D, bool BF16, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_kernel(FwdArgs a) {
  using MM = Mma16<BF16>;
  using op_t = typename MM::op_t;
  using el_t = typename MM::el_t;
  constexpr int KSTR = D + 16;   // bytes per K row in LDS
  constexpr int VSTR = kKT + 4;  // elements per V^T row in LDS
  constexpr int KS = D / 32;     // 32-deep k-steps of the INT8 product
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) int8_t k_lds[kKT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VSTR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work item -------------------------------------------------------------
  const int nheads = a.B * a.Hq;
  const int slot = blockIdx.x % nheads;
  const int rank = blockIdx.x / nheads;
  const int nkvu = a.B * a.Hkv;
  const int kvu = slot % nkvu;         // b * Hkv + hk: consecutive blocks, distinct XCDs
  const int g = slot / nkvu;
  const int b = kvu / a.Hkv;
  const int hk = kvu % a.Hkv;
  const int hq = hk * a.group + g;
  const int i = CAUSAL ? (a.nqb - 1 - rank) : rank;
  const size_t bhq = (size_t)b * a.Hq + hq;
  const int row0 = i * kQBlock + wave * 64;  // first query row of this wave

  // ---- Q fragments (B operand of S^T = K Q^T) ---------------------------------
  v4i qf[2][KS];
  {
    const int8_t* qg = a.q_i8 + (bhq * a.N + row0) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const v4i*>(qg + (size_t)(32 * qb + l32) * D + 32 * ks + 16 * h);
  }
  const float alpha_q = a.q_scale[bhq * a.nqb + i] * a.c;

  v16f acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][qb][r] = 0.0f;
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.0f, 0.0f};  // this lane's half of the row sum

  int ntiles;
  const int32_t* klist = nullptr;
  if constexpr (SPARSE) {
    ntiles = min(a.kv_cnt[bhq * a.nqb + i], a.max_keep);
    klist = a.kv_idx + (bhq * a.nqb + i) * a.max_keep;
  } else {
    ntiles = CAUSAL ? 2 * i + 2 : a.nkb;
  }
  const int last_tile_wave = row0 / kKT;  // causal: last tile this wave sees (its diagonal)
  const size_t kv_row0 = (size_t)kvu * a.N;

  for (int it = 0; it < ntiles; ++it) {
    const int t = SPARSE ? klist[it] : it;
    if (SPARSE) {
      // ignore entries outside the block range or past the causal range
      if (t < 0 || t >= a.nkb) continue;
      if (CAUSAL && t * kKT > i * kQBlock + kQBlock - 1) continue;
    }
    __syncthreads();  // previous tile's LDS readers are done
    {
      const int8_t* kg = a.k_i8 + (kv_row0 + (size_t)t * kKT) * D;
      constexpr int CPR = D / 16;
      for (int c = threadIdx.x; c < kKT * CPR; c += kThreads) {
        const int r = c / CPR, col = c % CPR;
        *reinterpret_cast<int4*>(&k_lds[r * KSTR + col * 16]) =
            *reinterpret_cast<const int4*>(kg + (size_t)r * D + col * 16);
      }
      const uint16_t* vg = a.v + (kv_row0 + (size_t)t * kKT) * D;
      constexpr int EPR = D / 8;
      for (int c = threadIdx.x; c < kKT * EPR; c += kThreads) {
        const int key = c / EPR, d0 = (c % EPR) * 8;
        const uint4 w = *reinterpret_cast<const uint4*>(vg + (size_t)key * D + d0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt_lds[(d0 + 2 * e) * VSTR + key] = (uint16_t)(ws[e] & 0xffffu);
          vt_lds[(d0 + 2 * e + 1) * VSTR + key] = (uint16_t)(ws[e] >> 16);
        }
      }
    }
    __syncthreads();
    if (CAUSAL && t > last_tile_wave) continue;  // wave-uniform: all keys masked
    const bool diag = CAUSAL && t == last_tile_wave;

    // ---- S^T = K Q^T (INT8) ---------------------------------------------------
    v16i sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v4i kf = *reinterpret_cast<const v4i*>(&k_lds[(kb * 32 + l32) * KSTR + 32 * ks + 16 * h]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[qb][ks], sacc[kb][qb], 0, 0, 0);
      }
    }

    // ---- online softmax, one query column per lane and block ------------------
    const float alpha = alpha_q * a.k_scale[(size_t)kvu * a.nkb + t];
    op_t pf[2][2][2];  // [kb][qb][half of the 32 keys]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float f[2][16];
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = (float)sacc[kb][qb][r];
          if (diag) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const int q = 32 * qb + l32;
            if (key > q) x = -__builtin_inff();
          }
          f[kb][r] = x;
          mx = __builtin_fmaxf(mx, x);
        }
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = __builtin_fmaxf(m_run[qb], mx * alpha);
      const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      const float corr = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
      m_run[qb] = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(f[kb][8 * half + e], alpha, -m_use));
            const el_t pe = (el_t)p;
            psum += (float)pe;
            pf[kb][qb][half][e] = pe;
          }
      l_run[qb] = l_run[qb] * corr + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][qb][r] *= corr;
    }

    // ---- O^T += V^T P^T (16-bit operands, fp32 accumulate) -------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint16_t* vr = &vt_lds[(db * 32 + l32) * VSTR + kb * 32 + 16 * half + 4 * h];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
          const v4i raw = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
          const op_t vf = __builtin_bit_cast(op_t, raw);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) acc[db][qb] = MM::mma(vf, pf[kb][qb][half], acc[db][qb]);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l, lse -------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int q = row0 + 32 * qb + l32;
    uint16_t* og = a.o + (bhq * a.N + q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        uint16_t e16[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const el_t y = (el_t)(acc[db][qb][4 * grp + e] * inv);
          e16[e] = __builtin_bit_cast(uint16_t, y);
        }
        uint2 w;
        w.x = (uint32_t)e16[0] | ((uint32_t)e16[1] << 16);
        w.y = (uint32_t)e16[2] | ((uint32_t)e16[3] << 16);
        *reinterpret_cast<uint2*>(og + db * 32 + 8 * grp + 4 * h) = w;
      }
    if (a.lse != nullptr && h == 0) {
      a.lse[bhq * a.N + q] =
          lt > 0.0f ? 0.69314718055994531f * (m_run[qb] + __builtin_log2f(lt)) : -__builtin_inff();
    }
  }
}

template <int D, bool BF16>
hipError_t launch_d(const FwdArgs& a, bool causal, bool sparse, hipStream_t stream) {
  const dim3 grid(a.B * a.Hq * a.nqb), block(kThreads);
  if (causal) {
    if (sparse)
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, true, false>), grid, block, 0, stream, a);
  } else {
    if (sparse)
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, const int8_t* q_i8, const float* q_scale,
                           const int8_t* k_i8, const float* k_scale, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, int max_keep, void* o,
                           float* lse, hipStream_t stream) {
  FwdArgs a;
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.group = s.Hq / s.Hkv;
  a.nqb = s.nqb();
  a.nkb = s.nkb();
  a.max_keep = max_keep;
  // the softmax temperature folded with the change to base 2, rounded once
  a.c = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d));
  const bool sparse = kv_idx != nullptr;
  if (s.d == 128)
    return s.bf16 ? launch_d<128, true>(a, s.causal, sparse, stream)
                  : launch_d<128, false>(a, s.causal, sparse, stream);
  return s.bf16 ? launch_d<64, true>(a, s.causal, sparse, stream)
                : launch_d<64, false>(a, s.causal, sparse, stream);
}

}  // namespace qattn
