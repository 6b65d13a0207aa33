// Quantized attention forward on gfx950 matrix cores.
//
// Work decomposition. A wave owns 32 query rows of one query head (one
// 32-column MFMA block). Dense: a workgroup of 8 waves takes g4 = 4, 2 or 1
// query heads of one kv head (the largest that divides the group size) times
// 8/g4 consecutive 32-row slabs, so all 8 waves share every K/V tile they
// stage (GQA group 4: four heads x the same 64 rows). Sparse: a workgroup of
// 4 waves takes one 128-row query block of one head; its kept list is the
// workgroup's tile list. Consecutive workgroups map to distinct kv heads, so
// blockIdx % 8 (the XCD) keeps each kv head on one XCD's L2; under causal
// masking the longest rows are dispatched first.
//
// Per 64-key tile (registers except the K/V staging):
//   S^T[key][q] = K_tile . Q^T       v_mfma_i32_32x32x32_i8, two 32-key blocks,
//                                    4 (d = 128) or 2 (d = 64) k-steps
//   online base-2 softmax on S^T     lane = query column; lanes l, l+32 hold the
//                                    two halves of its 32 keys per block
//   O^T[d][q] += V^T . P^T           v_mfma_f32_32x32x16_{bf16,f16}
// The transposed products make the INT8 accumulator layout (lane = column,
// registers = rows) the B-operand layout of the 16-bit MFMA: P never leaves
// registers. K and V are staged row-major in LDS by direct global->LDS loads
// (global_load_lds_dwordx4: one wave instruction fills 1 KB); each row's
// 16-byte slots are XOR-swizzled by the row index so that the 16-byte K
// fragment reads and the 8-byte transposing V reads are free of bank
// conflicts. The V^T operand comes from ds_read_b64_tr_b16, which hands each
// lane 4 consecutive keys of one channel.
//
// Pipeline (triple buffers, one barrier per tile): iteration t issues the
// asynchronous loads of V(t+1) and K(t+3), computes the softmax of tile t, a
// P V product and S of tile t+1, then waits for everything but its K loads.
// In 8-wave workgroups the waves sharing a SIMD take opposite ping-pong roles
// (see the pipeline below) so that VALU and matrix work overlap.
//
// Online softmax reference: a row's exponent reference m moves only when the
// tile's running max exceeds it by more than kTau (log2 units); otherwise P is
// taken against the stale reference (P <= 2^kTau) and the accumulator is not
// rescaled. The move test is wave-uniform, so the rescale is skipped for the
// whole wave in the common case.
#include "../../include/qattn.h"
#include "device_util.h"
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kKT = 64;             // keys per tile
constexpr float kTau = QATTN_SOFTMAX_REF_THRESHOLD;  // log2 units
constexpr int kMaxSparseTiles = 2048;

template <bool BF16>
struct Mma16;

template <>
struct Mma16<true> {
  typedef v8bf op_t;
  typedef v2bf pair_t;
  typedef __bf16 el_t;
  static __device__ __forceinline__ v16f mma(op_t a, op_t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // sum of the two 16-bit values of a pair, accumulated in fp32
  static __device__ __forceinline__ float sum2(pair_t p, float acc) {
    const pair_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
};

template <>
struct Mma16<false> {
  typedef v8h op_t;
  typedef v2h pair_t;
  typedef _Float16 el_t;
  static __device__ __forceinline__ v16f mma(op_t a, op_t b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum2(pair_t p, float acc) {
    const pair_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(p, one, acc, false);
  }
};

__device__ __forceinline__ v4s lds_read_tr16(const int8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}

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
  int B, Hq, Hkv, N, group, g4, nqb, nkb, max_keep;
  float c;  // fl32(log2(e) / sqrt(d))
};

template <int D>
struct Geo {
  static constexpr int KROW = D;           // K row in LDS (bytes, unpadded)
  static constexpr int VROW = 2 * D;       // V row in LDS (bytes, unpadded)
  static constexpr int KBUF = kKT * KROW;
  static constexpr int VBUF = kKT * VROW;
  static constexpr int KS = D / 32;        // 32-deep k-steps of the INT8 product
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int KSLOTS = D / 16;    // 16-byte slots per K row
  static constexpr int VSLOTS = D / 8;     // 16-byte slots per V row
  // The LDS has 64 banks of 4 bytes (256 bytes per cycle): a 16-byte read is
  // served 16 lanes at a time, an 8-byte transposing read 32 lanes at a time.
  // Swizzle of a K row: slot s of row r holds chunk s ^ kswz(r), so the 16
  // consecutive rows of one 16-lane phase (same chunk) cover all 64 banks.
  static __device__ __forceinline__ int kswz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  // Swizzle of a V row: the 32 lanes of one phase read 4 rows x 2 channel
  // halves x 32 bytes; these 8 pieces land on disjoint bank groups.
  static __device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane (global_load_lds_dwordx4, LDS base in M0).
__device__ __forceinline__ void lds_dma16(const void* g, int8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds_wave_base, 16, 0, 0);
}

template <int D, bool BF16, bool CAUSAL, bool SPARSE, int QB, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_kernel(FwdArgs a) {
  using MM = Mma16<BF16>;
  using op_t = typename MM::op_t;
  using pair_t = typename MM::pair_t;
  using el_t = typename MM::el_t;
  using G = Geo<D>;
  constexpr int RW = 32 * QB;
  constexpr int KPIECES = G::KBUF / 1024;  // 1 KB direct loads per K tile
  constexpr int VPIECES = G::VBUF / 1024;
  // three K and three V buffers as distinct objects, always named with
  // compile-time indices: the compiler can then tell that an LDS read of one
  // buffer does not depend on the DMA loads still landing in another, and
  // waits only for the loads of the buffer it reads
  __shared__ __attribute__((aligned(16))) int8_t k_lds0[G::KBUF];
  __shared__ __attribute__((aligned(16))) int8_t k_lds1[G::KBUF];
  __shared__ __attribute__((aligned(16))) int8_t k_lds2[G::KBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds0[G::VBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds1[G::VBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds2[G::VBUF];
  __shared__ int16_t tile_list[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int n_list;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int nkvu = a.B * a.Hkv;

  // ---- work item ---------------------------------------------------------------
  int kvu, hq, row0, wg_last_row, qblk;
  if constexpr (SPARSE) {
    const int nheads = a.B * a.Hq;
    const int slot = blockIdx.x % nheads;
    const int rank = blockIdx.x / nheads;
    kvu = slot % nkvu;
    const int g = slot / nkvu;
    hq = (kvu % a.Hkv) * a.group + g;
    qblk = CAUSAL ? (a.nqb - 1 - rank) : rank;
    row0 = qblk * kQBlock + RW * wave;
    wg_last_row = qblk * kQBlock + kQBlock - 1;
  } else {
    const int g4 = a.g4;
    const int rows_wg = RW * (NW / g4);
    const int nrc = (a.N + rows_wg - 1) / rows_wg;
    const int nsub = a.group / g4;
    const int nslot = nkvu * nsub;
    const int slot = blockIdx.x % nslot;
    const int rank = blockIdx.x / nslot;
    kvu = slot % nkvu;
    const int hs = slot / nkvu;
    const int rc = CAUSAL ? (nrc - 1 - rank) : rank;
    hq = (kvu % a.Hkv) * a.group + hs * g4 + wave % g4;
    row0 = rc * rows_wg + RW * (wave / g4);
    wg_last_row = min(a.N, rc * rows_wg + rows_wg) - 1;
    qblk = row0 / kQBlock;
  }
  const int b = kvu / a.Hkv;
  const size_t bhq = (size_t)b * a.Hq + hq;
  const bool wave_live = row0 < a.N;  // wave-uniform
  const size_t kv_row0 = (size_t)kvu * a.N;

  // ---- tile list -----------------------------------------------------------------
  int ntiles;
  if constexpr (SPARSE) {
    if (wave == 0) {
      const int cnt = min(a.kv_cnt[bhq * a.nqb + qblk], min(a.max_keep, kMaxSparseTiles));
      const int32_t* src = a.kv_idx + (bhq * a.nqb + qblk) * a.max_keep;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int n = 0;
      for (int e0 = 0; e0 < cnt; e0 += 64) {
        const int e = e0 + lane;
        const int t = e < cnt ? src[e] : -1;
        const bool ok = t >= 0 && t < a.nkb && (!CAUSAL || t * kKT <= wg_last_row);
        const uint64_t bal = __ballot(ok);
        if (ok) tile_list[n + __popcll(bal & lt)] = (int16_t)t;
        n += __popcll(bal);
      }
      if (lane == 0) n_list = n;
    }
    __syncthreads();
    ntiles = n_list;
  } else {
    ntiles = CAUSAL ? wg_last_row / kKT + 1 : a.nkb;
  }
  auto tile_of = [&](int it) -> int {
    if constexpr (SPARSE) return tile_list[it];
    else return it;
  };
  // causal: a tile is needed while its first key is at or before the wave's
  // last row; it needs masking when it reaches past the wave's first row
  auto wave_needs = [&](int t) -> bool { return wave_live && (!CAUSAL || t * kKT <= row0 + RW - 1); };

  // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------------
  v4i qf[QB][G::KS];
  if (wave_live) {
    const int8_t* qg = a.q_i8 + (bhq * a.N + row0) * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const v4i*>(qg + (size_t)(32 * qb + l32) * D + 32 * ks + 16 * h);
  }
  const float alpha_q = wave_live ? a.q_scale[bhq * a.nqb + qblk] * a.c : 0.0f;
  // k_scale through the constant address space: a uniform index makes this a
  // scalar load (counted by lgkmcnt), so it never waits behind the in-flight
  // vector (LDS DMA) loads of later tiles
  const __attribute__((address_space(4))) float* kscale =
      (const __attribute__((address_space(4))) float*)(a.k_scale + (size_t)kvu * a.nkb);

  v16f acc[G::DB][QB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][qb][r] = 0.0f;
  float m_ref[QB], l_run[QB];  // l_run: this lane's half of the row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -__builtin_inff();
    l_run[qb] = 0.0f;
  }

  // ---- staging: direct global -> LDS, 1 KB per wave instruction -------------------
  // In piece p, lane l writes slot l % SLOTS of row p*(1024/ROW) + l / SLOTS,
  // so it fetches that row's global chunk (slot ^ swizzle(row)).
  auto k_src_off = [&](int piece) {
    const int r = piece * (1024 / G::KROW) + lane / G::KSLOTS;
    return r * G::KROW + (((lane % G::KSLOTS) ^ G::kswz(r)) * 16);
  };
  auto v_src_off = [&](int piece) {
    const int r = piece * (1024 / G::VROW) + lane / G::VSLOTS;
    return r * G::VROW + (((lane % G::VSLOTS) ^ G::vswz(r)) * 16);
  };
  auto load_k = [&](int t, int8_t* buf) {
    const int8_t* src = a.k_i8 + (kv_row0 + (size_t)t * kKT) * D;
#pragma unroll
    for (int piece = wave; piece < KPIECES; piece += NW)
      lds_dma16(src + k_src_off(piece), buf + piece * 1024);
  };
  auto load_v = [&](int t, int8_t* buf) {
    const int8_t* src = reinterpret_cast<const int8_t*>(a.v + (kv_row0 + (size_t)t * kKT) * D);
#pragma unroll
    for (int piece = wave; piece < VPIECES; piece += NW)
      lds_dma16(src + v_src_off(piece), buf + piece * 1024);
  };
  // loads one wave issues per K / V tile (the fewest over the waves: waiting
  // for that many to remain outstanding is safe for every wave)
  constexpr int KPW = KPIECES / NW;
  auto wait_all = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // workgroup barrier without the compiler's implied full memory wait: the
  // LDS DMA loads this wave still has in flight target buffers nobody reads
  // before the next barrier, and its own LDS reads are drained here
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // wait for every load of this wave except this iteration's K loads (issued
  // last) when there are some
  auto wait_older = [&](bool k_pending, bool) {
    if (k_pending && KPW > 0) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KPW) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // ---- compute helpers -----------------------------------------------------------
  // K fragment (key row kb*32 + l32, chunk 2*ks + h), swizzled; kswz only
  // depends on the row's low five bits, so kb*32 keeps it
  int k_frag_off[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) k_frag_off[ks] = l32 * G::KROW + (((2 * ks + h) ^ G::kswz(l32)) * 16);
  // S is accumulated on top of the integer bit pattern of kMagic = 1.5 * 2^23:
  // the int32 result M + S read as a float is exactly kMagic + S (|S| <=
  // 128 * 127^2 < 2^22), so the softmax gets floats without a conversion and
  // recovers S exactly with one subtraction.
  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = 0x4B400000;
  auto qk = [&](const int8_t* kbuf, v16i (&s)[2][QB]) {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v4i kf = *reinterpret_cast<const v4i*>(kbuf + kb * 32 * G::KROW + k_frag_off[ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (ks == 0) {
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[qb][ks], magic, 0, 0, 0);
          } else {
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[qb][ks], s[kb][qb], 0, 0, 0);
          }
        }
      }
    }
  };

  // softmax of one tile, one 32-query block at a time: S (kMagic-biased
  // floats) -> P packed in the B-operand layout of the P V product
  constexpr float kMagic = 12582912.0f;
  auto softmax = [&](const v16i (&s)[2][QB], int t, op_t (&pf)[2][QB][2]) {
    const float alpha = alpha_q * kscale[__builtin_amdgcn_readfirstlane(t)];
    const bool diag = CAUSAL && t * kKT + kKT - 1 > row0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float f[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // copy the element out first: __builtin_bit_cast of a vector
          // element reads the vector's first element
          const int si = s[kb][qb][r];
          f[16 * kb + r] = __builtin_bit_cast(float, si);
        }
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t * kKT + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > row0 + 32 * qb + l32) f[16 * kb + r] = -__builtin_inff();
          }
      }
      // row max: a max3 tree over the lane's 32 keys, then the other half-row
      float m8[11];
#pragma unroll
      for (int j = 0; j < 10; ++j) m8[j] = __builtin_fmaxf(__builtin_fmaxf(f[3 * j], f[3 * j + 1]), f[3 * j + 2]);
      m8[10] = __builtin_fmaxf(f[30], f[31]);
      const float m4a = __builtin_fmaxf(__builtin_fmaxf(m8[0], m8[1]), m8[2]);
      const float m4b = __builtin_fmaxf(__builtin_fmaxf(m8[3], m8[4]), m8[5]);
      const float m4c = __builtin_fmaxf(__builtin_fmaxf(m8[6], m8[7]), m8[8]);
      const float m4d = __builtin_fmaxf(m8[9], m8[10]);
      float mx = __builtin_fmaxf(__builtin_fmaxf(m4a, m4b), __builtin_fmaxf(m4c, m4d));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, mx),
                                                         __builtin_bit_cast(int, mx), false, false);
        mx = __builtin_fmaxf(__builtin_bit_cast(float, (int)sw[0]), __builtin_bit_cast(float, (int)sw[1]));
      }
      // fl32(max S * alpha): the subtraction is exact (same binade)
      const float mc = __builtin_fmaxf(m_ref[qb], (mx - kMagic) * alpha);
      const bool move = mc > m_ref[qb] + kTau;
      if (__ballot(move) != 0) {
        float corr = 1.0f;
        if (move) {
          corr = (m_ref[qb] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_ref[qb] - mc);
          m_ref[qb] = mc;
        }
        l_run[qb] *= corr;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][qb][r] *= corr;
      }
      const float m_use = (m_ref[qb] == -__builtin_inff()) ? 0.0f : m_ref[qb];
      float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          op_t pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = f[16 * kb + 8 * half + e] - kMagic;  // exact: S as a float
            pk[e] = (el_t)__builtin_amdgcn_exp2f(__builtin_fmaf(d, alpha, -m_use));
          }
          // four independent fp32 partial sums of the rounded P
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const pair_t pr = {pk[2 * w], pk[2 * w + 1]};
            lsum[w] = MM::sum2(pr, lsum[w]);
          }
          pf[kb][qb][half] = pk;
        }
      l_run[qb] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    }
  };

  // transposing V reads: 16-lane group g = lane/16 reads key rows
  // k0 + 4*(g/2) + (lane%16)/4 and the 32 bytes of channels
  // 32*db + 16*(g%2) + [0, 16); lane j of the group takes 8 of them. k0 is a
  // multiple of 8, so the row bits the swizzle reads depend on the lane only.
  const int grp = lane >> 4;
  const int vr_lane = 4 * (grp >> 1) + ((lane >> 2) & 3);
  int v_frag_off[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) {
    const int slot = 4 * db + 2 * (grp & 1) + ((lane & 3) >> 1);
    v_frag_off[db] = vr_lane * G::VROW + ((slot ^ G::vswz(vr_lane)) * 16) + 8 * (lane & 1);
  }
  auto pv = [&](const int8_t* vbuf, const op_t (&pf)[2][QB][2]) {
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int8_t* p = vbuf + (kb * 32 + 16 * half) * G::VROW + v_frag_off[db];
          const v4s lo = lds_read_tr16(p);
          const v4s hi = lds_read_tr16(p + 8 * G::VROW);
          const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const op_t vf = __builtin_bit_cast(op_t, both);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[db][qb] = MM::mma(vf, pf[kb][qb][half], acc[db][qb]);
        }
  };

  // ---- pipeline ---------------------------------------------------------------------
  if (ntiles > 0) load_v(tile_of(0), v_lds0);
  if (ntiles > 0) load_k(tile_of(0), k_lds0);
  if (ntiles > 1) load_k(tile_of(1), k_lds1);
  if (ntiles > 2) load_k(tile_of(2), k_lds2);
  wait_all();
  __syncthreads();

  // Ping-pong roles (dense, 8 waves: waves w and w+4 share a SIMD). Role A
  // runs softmax(t), P V(t), S(t+1); role B runs P V(t-1), softmax(t), S(t+1),
  // so on each SIMD one wave's softmax (VALU) runs against the other's matrix
  // products. B keeps P(t-1) across the barrier and finishes with P V(last).
  constexpr bool kPingPong = !SPARSE && NW == 8;
  const bool role_b = kPingPong && wave >= 4;

  v16i s[2][QB];
  op_t p_prev[2][QB][2];
  bool have_prev = false;
  if (ntiles > 0 && wave_needs(tile_of(0))) qk(k_lds0, s);
  // one tile. Buffers: tile j's K and V live in buffer j % 3. The loads of
  // iteration it go to V(it+1) -> (it+1) % 3 (last read by role B at it-1)
  // and K(it+3) -> it % 3 (K(it) was last read at it-1); V is issued first so
  // that waiting for it leaves only this iteration's K loads in flight.
  auto step = [&](int it, int8_t* k_cur, int8_t* k_next, const int8_t* v_prev,
                  const int8_t* v_cur, int8_t* v_next) {
    const int t = tile_of(it);
    const bool pre_v = it + 1 < ntiles;
    const bool pre_k = it + 3 < ntiles;
    if (pre_v) load_v(tile_of(it + 1), v_next);
    if (pre_k) load_k(tile_of(it + 3), k_cur);
    const bool need = wave_needs(t);
    if (role_b) {
      if (have_prev) pv(v_prev, p_prev);
      op_t pf[2][QB][2];
      if (need) softmax(s, t, pf);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < QB; ++y)
#pragma unroll
          for (int z = 0; z < 2; ++z) p_prev[x][y][z] = pf[x][y][z];
      have_prev = need;
    } else if (need) {
      op_t pf[2][QB][2];
      softmax(s, t, pf);
      pv(v_cur, pf);
    }
    if (it + 1 < ntiles && wave_needs(tile_of(it + 1))) qk(k_next, s);
    wait_older(pre_k, false);
    barrier();
  };
  int it = 0;
  for (; it + 3 <= ntiles; it += 3) {
    step(it, k_lds0, k_lds1, v_lds2, v_lds0, v_lds1);
    step(it + 1, k_lds1, k_lds2, v_lds0, v_lds1, v_lds2);
    step(it + 2, k_lds2, k_lds0, v_lds1, v_lds2, v_lds0);
  }
  if (it < ntiles) step(it, k_lds0, k_lds1, v_lds2, v_lds0, v_lds1);
  if (it + 1 < ntiles) step(it + 1, k_lds1, k_lds2, v_lds0, v_lds1, v_lds2);
  if (have_prev) {
    // role B: the last tile's P V; its V buffer is (ntiles - 1) % 3
    const int lb = (ntiles - 1) % 3;
    if (lb == 0) pv(v_lds0, p_prev);
    else if (lb == 1) pv(v_lds1, p_prev);
    else pv(v_lds2, p_prev);
  }

  // ---- epilogue: O = acc / l, lse --------------------------------------------------
  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int q = row0 + 32 * qb + l32;
    uint16_t* og = a.o + (bhq * a.N + q) * D;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint16_t e16[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const el_t y = (el_t)(acc[db][qb][4 * g + e] * inv);
          e16[e] = __builtin_bit_cast(uint16_t, y);
        }
        uint2 w;
        w.x = (uint32_t)e16[0] | ((uint32_t)e16[1] << 16);
        w.y = (uint32_t)e16[2] | ((uint32_t)e16[3] << 16);
        *reinterpret_cast<uint2*>(og + db * 32 + 8 * g + 4 * h) = w;
      }
    if (a.lse != nullptr && h == 0) {
      a.lse[bhq * a.N + q] =
          lt > 0.0f ? 0.69314718055994531f * (m_ref[qb] + __builtin_log2f(lt)) : -__builtin_inff();
    }
  }
}

#ifndef QATTN_NW_DENSE
#define QATTN_NW_DENSE 8
#endif
#ifndef QATTN_QB
#define QATTN_QB 1
#endif

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_dc(const FwdArgs& a, bool sparse, hipStream_t stream) {
  constexpr int QB = QATTN_QB;          // 32-query blocks per wave
  constexpr int WPE = QB == 1 ? 2 : 1;  // waves per SIMD
  constexpr int NW_DENSE = QATTN_NW_DENSE;
  constexpr int NW_SPARSE = 128 / (32 * QB);
  if (sparse) {
    const dim3 grid(a.B * a.Hq * a.nqb);
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, QB, NW_SPARSE, WPE>), grid,
                       dim3(NW_SPARSE * 64), 0, stream, a);
  } else {
    const int rows_wg = 32 * QB * (NW_DENSE / a.g4);
    const int nrc = (a.N + rows_wg - 1) / rows_wg;
    const dim3 grid(a.B * a.Hkv * (a.group / a.g4) * nrc);
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, false, QB, NW_DENSE, WPE>), grid,
                       dim3(NW_DENSE * 64), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(const FwdArgs& a, bool causal, bool sparse, hipStream_t stream) {
  return causal ? launch_dc<D, BF16, true>(a, sparse, stream)
                : launch_dc<D, BF16, false>(a, sparse, stream);
}

}  // namespace

int fwd_max_sparse_tiles() { return kMaxSparseTiles; }

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
  a.g4 = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0) ? 2 : 1;
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
