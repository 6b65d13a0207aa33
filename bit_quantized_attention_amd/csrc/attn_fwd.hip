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
// Pipeline (three K/V buffers, one barrier per tile): each wave runs S, the
// softmax and P V of its tile in sequence; the waves sharing a SIMD overlap
// each other's matrix and vector work. The loads of the tile two ahead go out
// once the current S products are queued. Dense workgroups keep each wave's Q
// fragments in LDS; every K tile carries its scale in a small tail of its LDS
// buffer (no scalar loads in the loop).
//
// Online softmax reference: a row's exponent reference m moves only when the
// tile's running max exceeds it by more than kTau (log2 units); otherwise P is
// taken against the stale reference (P <= 2^kTau) and the accumulator is not
// rescaled. The move test is wave-uniform, so the rescale is skipped for the
// whole wave in the common case.
#include <climits>
#include <type_traits>

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
// 4 bytes per lane (global_load_lds_dword), LDS destination lds_base + 4 * lane
__device__ __forceinline__ void lds_dma4(const void* g, int8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds_base, 4, 0, 0);
}

__device__ __forceinline__ void lds_dma16(const void* g, int8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds_wave_base, 16, 0, 0);
}

// compile-time loop: f(integral_constant<int, I>) for I in [I0, N)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int D, bool BF16, bool CAUSAL, bool SPARSE, int QB, int NW, int WPE, int NBUF>
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
  // NBUF K and NBUF V buffers as distinct objects, always named with
  // compile-time indices: the compiler can then tell that an LDS read of one
  // buffer does not depend on the DMA loads still landing in another, and
  // waits only for the loads of the buffer it reads
  static_assert(NBUF == 3 || NBUF == 4, "three or four staging buffers");
  __shared__ __attribute__((aligned(16))) int8_t k_lds0[G::KBUF + 256];
  __shared__ __attribute__((aligned(16))) int8_t k_lds1[G::KBUF + 256];
  __shared__ __attribute__((aligned(16))) int8_t k_lds2[G::KBUF + 256];
  __shared__ __attribute__((aligned(16))) int8_t k_lds3[NBUF == 4 ? G::KBUF + 256 : 16];
  __shared__ __attribute__((aligned(16))) int8_t v_lds0[G::VBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds1[G::VBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds2[G::VBUF];
  __shared__ __attribute__((aligned(16))) int8_t v_lds3[NBUF == 4 ? G::VBUF : 16];
  auto kbuf = [&](auto i) -> int8_t* {
    constexpr int j = decltype(i)::value % NBUF;
    if constexpr (j == 0) return k_lds0;
    else if constexpr (j == 1) return k_lds1;
    else if constexpr (j == 2) return k_lds2;
    else return k_lds3;
  };
  auto vbuf = [&](auto i) -> int8_t* {
    constexpr int j = decltype(i)::value % NBUF;
    if constexpr (j == 0) return v_lds0;
    else if constexpr (j == 1) return v_lds1;
    else if constexpr (j == 2) return v_lds2;
    else return v_lds3;
  };
  // Dense workgroups keep each wave's Q fragments in LDS (same swizzle as a
  // K block) and read them per tile: that frees the 16 registers they would
  // hold for the whole kernel. Sparse workgroups keep them in registers (their
  // LDS budget allows two workgroups per CU).
  constexpr bool QL = !SPARSE;
  static_assert(!QL || QB == 1, "Q in LDS takes one 32-row block per wave");
  __shared__ __attribute__((aligned(16))) int8_t q_lds[QL ? NW * 32 * D : 16];
  __shared__ int16_t tile_list[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int n_list, n_list_plain;

  const int lane = threadIdx.x & 63;
  // wave index as a uniform (scalar) value: branches on it stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int nkvu = a.B * a.Hkv;

  // ---- work item ---------------------------------------------------------------
  int kvu, hq, row0, wg_row0, wg_last_row, qblk;
  if constexpr (SPARSE) {
    const int nheads = a.B * a.Hq;
    const int slot = blockIdx.x % nheads;
    const int rank = blockIdx.x / nheads;
    kvu = slot % nkvu;
    const int g = slot / nkvu;
    hq = (kvu % a.Hkv) * a.group + g;
    qblk = CAUSAL ? (a.nqb - 1 - rank) : rank;
    row0 = qblk * kQBlock + RW * wave;
    wg_row0 = qblk * kQBlock;
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
    wg_row0 = rc * rows_wg;
    wg_last_row = min(a.N, rc * rows_wg + rows_wg) - 1;
    qblk = row0 / kQBlock;
  }
  const int b = kvu / a.Hkv;
  const size_t bhq = (size_t)b * a.Hq + hq;
  const bool wave_live = row0 < a.N;  // wave-uniform
  const size_t kv_row0 = (size_t)kvu * a.N;

  // ---- tile list -----------------------------------------------------------------
  // Under causal masking a tile needs the per-element mask when its last key
  // lies past the workgroup's first row. Those tiles come last: n_plain
  // unmasked tiles, then the masked ones (for a valid kept list, which is
  // ascending, this is the given order).
  auto masked = [&](int t) -> bool { return CAUSAL && t * kKT + kKT - 1 > wg_row0; };
  int ntiles, n_plain;
  if constexpr (SPARSE) {
    if (wave == 0) {
      const int cnt = min(a.kv_cnt[bhq * a.nqb + qblk], min(a.max_keep, kMaxSparseTiles));
      const int32_t* src = a.kv_idx + (bhq * a.nqb + qblk) * a.max_keep;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int n = 0;
      for (int pass = 0; pass < 2; ++pass) {
        for (int e0 = 0; e0 < cnt; e0 += 64) {
          const int e = e0 + lane;
          const int t = e < cnt ? src[e] : -1;
          const bool ok = t >= 0 && t < a.nkb && (!CAUSAL || t * kKT <= wg_last_row) &&
                          (masked(t) == (pass == 1));
          const uint64_t bal = __ballot(ok);
          if (ok) tile_list[n + __popcll(bal & lt)] = (int16_t)t;
          n += __popcll(bal);
        }
        if (pass == 0 && lane == 0) n_list_plain = n;
      }
      if (lane == 0) n_list = n;
    }
    __syncthreads();
    ntiles = n_list;
    n_plain = n_list_plain;
  } else {
    ntiles = CAUSAL ? wg_last_row / kKT + 1 : a.nkb;
    n_plain = CAUSAL ? min(ntiles, (wg_row0 + 1) / kKT) : ntiles;
  }
  auto tile_of = [&](int it) -> int {
    if constexpr (SPARSE) return tile_list[it];
    else return it;
  };

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
  const float* kscale = a.k_scale + (size_t)kvu * a.nkb;

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
  // (unsigned 32-bit offsets from a uniform base: the loads then use the
  // scalar-base addressing form instead of per-lane 64-bit adds)
  auto k_src_off = [&](int piece) -> uint32_t {
    const int r = piece * (1024 / G::KROW) + lane / G::KSLOTS;
    return (uint32_t)(r * G::KROW + (((lane % G::KSLOTS) ^ G::kswz(r)) * 16));
  };
  auto v_src_off = [&](int piece) -> uint32_t {
    const int r = piece * (1024 / G::VROW) + lane / G::VSLOTS;
    return (uint32_t)(r * G::VROW + (((lane % G::VSLOTS) ^ G::vswz(r)) * 16));
  };
  // Every wave issues the same fixed number of 1 KB loads per tile (KPW, VPW):
  // piece (wave + NW*j) % PIECES. When a tile has fewer pieces than the group
  // has waves, several waves load the same piece (identical bytes).
  // wave w loads pieces w, w+NW, ... (mod the piece count): every piece is
  // covered, and a few are loaded twice (identical bytes) when the piece count
  // is not a multiple of the wave count
  constexpr int KPW = (KPIECES + NW - 1) / NW;
  constexpr int VPW = (VPIECES + NW - 1) / NW;
  // The K tile's scale rides along into the 256-byte tail of its buffer (all
  // 64 lanes load the same word), so the softmax reads it from LDS: no
  // scalar load, whose out-of-order return would make every LDS wait a full
  // wait.
  auto load_k = [&](int t, int8_t* buf) {
    const int8_t* src = a.k_i8 + (kv_row0 + (size_t)t * kKT) * D;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int piece = (wave + NW * j) % KPIECES;
      lds_dma16(src + k_src_off(piece), buf + piece * 1024);
    }
    lds_dma4(kscale + t, buf + G::KBUF);
  };
  auto tile_kscale = [&](const int8_t* buf) {
    return *reinterpret_cast<const float*>(buf + G::KBUF);
  };
  auto load_v = [&](int t, int8_t* buf) {
    const int8_t* src = reinterpret_cast<const int8_t*>(a.v + (kv_row0 + (size_t)t * kKT) * D);
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int piece = (wave + NW * j) % VPIECES;
      lds_dma16(src + v_src_off(piece), buf + piece * 1024);
    }
  };
  // Waits go through the s_waitcnt builtin (not inline asm) so that the
  // compiler's own wait insertion knows which loads have already landed and
  // adds no full wait in front of the LDS reads. Encoding (gfx9): vmcnt in
  // bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; unused fields at maximum.
  auto wait_all = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };
  // workgroup barrier without the compiler's implied full memory wait: the
  // LDS DMA loads this wave still has in flight target buffers nobody reads
  // before the next barrier, and its own LDS reads are drained here
  auto barrier = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  // ---- compute helpers -----------------------------------------------------------
  // K fragment (key row kb*32 + l32, chunk 2*ks + h), swizzled; kswz only
  // depends on the row's low five bits, so kb*32 keeps it
  int k_frag_off[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) k_frag_off[ks] = l32 * G::KROW + (((2 * ks + h) ^ G::kswz(l32)) * 16);
  const int8_t* q_wave = q_lds + (QL ? wave * 32 * D : 0);
  auto qk = [&](const int8_t* kbuf, v16i (&s)[2][QB]) {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      v4i qv[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (QL) qv[qb] = *reinterpret_cast<const v4i*>(q_wave + k_frag_off[ks]);
        else qv[qb] = qf[qb][ks];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v4i kf = *reinterpret_cast<const v4i*>(kbuf + kb * 32 * G::KROW + k_frag_off[ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (ks == 0) {
            const v16i zero = {};
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qv[qb], zero, 0, 0, 0);
          } else {
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qv[qb], s[kb][qb], 0, 0, 0);
          }
        }
      }
    }
  };

  // softmax of one tile, one 32-query block at a time: S (exact int32) -> P
  // packed in the B-operand layout of the P V product. It moves the exponent
  // reference, rescales l and returns the accumulator's rescale factor corr (1
  // where the reference stayed; any_move says whether any row moved); the
  // caller applies corr to acc before this tile's P V. The row max is an
  // integer max3 tree (no NaN handling). With MASKED (causal tiles reaching
  // past the workgroup's first row), element (kb, r), which holds key
  // t*64 + 4h + off, is dropped when off > lim.
  auto softmax = [&](auto masked_c, const v16i (&s)[2][QB], float alpha, int t,
                     op_t (&pf)[2][QB][2], float (&corr)[QB], bool& any_move) {
    constexpr bool MASKED = decltype(masked_c)::value;
    any_move = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int lim = (row0 + 32 * qb + l32) - (t * kKT + 4 * h);
      int si[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          const int x = s[kb][qb][r];
          si[16 * kb + r] = (MASKED && off > lim) ? INT_MIN : x;
        }
      // row max: a max3 tree over the lane's 32 keys, then the other half-row
      int m8[11];
#pragma unroll
      for (int j = 0; j < 10; ++j) m8[j] = max(max(si[3 * j], si[3 * j + 1]), si[3 * j + 2]);
      m8[10] = max(si[30], si[31]);
      const int m4a = max(max(m8[0], m8[1]), m8[2]);
      const int m4b = max(max(m8[3], m8[4]), m8[5]);
      const int m4c = max(max(m8[6], m8[7]), m8[8]);
      const int m4d = max(m8[9], m8[10]);
      int mxi = max(max(m4a, m4b), max(m4c, m4d));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(mxi, mxi, false, false);
        mxi = max((int)sw[0], (int)sw[1]);
      }
      // fl32(max S * alpha) (S converts exactly: |S| < 2^24); in a fully
      // masked row every P is dropped below whatever the reference is
      const float mx = (float)mxi * alpha;
      const float mc = __builtin_fmaxf(m_ref[qb], mx);
      const bool move = mc > m_ref[qb] + kTau;
      any_move |= __ballot(move) != 0;
      const float m_old = m_ref[qb];
      corr[qb] = move ? (m_old == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_old - mc)) : 1.0f;
      m_ref[qb] = move ? mc : m_old;
      const float m_use = (m_ref[qb] == -__builtin_inff()) ? 0.0f : m_ref[qb];
      float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          op_t pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 16 * kb + 8 * half + e;
            const int off = kb * 32 + 8 * ((8 * half + e) >> 2) + (e & 3);
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf((float)si[i], alpha, -m_use));
            if constexpr (MASKED) pe = off > lim ? 0.0f : pe;
            pk[e] = (el_t)pe;
          }
          // four independent fp32 partial sums of the rounded P
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const pair_t pr = {pk[2 * w], pk[2 * w + 1]};
            lsum[w] = MM::sum2(pr, lsum[w]);
          }
          pf[kb][qb][half] = pk;
        }
      l_run[qb] = l_run[qb] * corr[qb] + ((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
    }
  };
  // acc *= corr, skipped by the whole wave when no row moved its reference
  auto rescale = [&](const float (&corr)[QB], bool any_move) {
    if (any_move) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][qb][r] *= corr[qb];
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
  // channel blocks innermost: consecutive matrix instructions update
  // different accumulators, so none waits for the one before it
  auto pv = [&](const int8_t* vbuf, const op_t (&pf)[2][QB][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
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
  // Tile j's K (with its scale) and V live in buffer j % NBUF. Iteration it
  // issues the loads of tile it+NBUF-1 into buffer (it-1) % NBUF (its last
  // readers ran in iteration it-1, before the previous barrier), computes
  // S = K Q^T, the softmax and P V of tile it, then waits until only the loads
  // of the last NBUF-2 iterations are in flight (tile it+1 has landed) and
  // passes the barrier. Each wave runs its tile in sequence; the other waves
  // on its SIMD fill the gaps (matrix and vector work overlap across waves).
  // Tiles past the end are clamped to the last tile (never read), so each
  // iteration issues the same loads. The loop is unrolled NBUF times so that
  // every buffer is named at compile time.
  static_for<0, NBUF - 1>([&](auto j) {
    const int tt = tile_of(min((int)j, ntiles - 1));
    load_k(tt, kbuf(j));
    load_v(tt, vbuf(j));
  });
  if constexpr (QL) {
    // this wave's Q fragments into its LDS slot (row l32, chunk 2ks+h,
    // swizzled like a K block)
    if (wave_live) {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        *reinterpret_cast<v4i*>(q_lds + wave * 32 * D + k_frag_off[ks]) = qf[0][ks];
    }
  }
  wait_all();
  __syncthreads();

  constexpr int kLoadsPerIt = KPW + 1 + VPW;  // K pieces, the K scale, V pieces
  constexpr auto vmcnt = [](int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); };
  static_assert((NBUF - 2) * kLoadsPerIt < 64, "vmcnt range");
  constexpr std::integral_constant<bool, true> kYes{};
  constexpr std::integral_constant<bool, false> kNo{};

  auto step = [&](auto jc, int it, auto masked_c) {
    constexpr int J = decltype(jc)::value;
    const std::integral_constant<int, J % NBUF> cur{};
    const std::integral_constant<int, (J + NBUF - 1) % NBUF> nxt{};
    // the next tile's loads go out once this tile's S products are queued
    const int tl = tile_of(min(it + NBUF - 1, ntiles - 1));
    if (wave_live) {
      const int t = tile_of(it);
      v16i s[2][QB];
      qk(kbuf(cur), s);
      load_k(tl, kbuf(nxt));
      load_v(tl, vbuf(nxt));
      op_t p[2][QB][2];
      float corr[QB];
      bool any_move;
      softmax(masked_c, s, alpha_q * tile_kscale(kbuf(cur)), t, p, corr, any_move);
      rescale(corr, any_move);
      pv(vbuf(cur), p);
    } else {
      load_k(tl, kbuf(nxt));
      load_v(tl, vbuf(nxt));
    }
    // The masked steps (a few per workgroup) wait for every load: any memory
    // instruction the compiler adds there is then covered too.
    if constexpr (decltype(masked_c)::value) {
      wait_all();
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt((NBUF - 2) * kLoadsPerIt));
    }
    barrier();
  };
  for (int base = 0; base < n_plain; base += NBUF) {
    static_for<0, NBUF>([&](auto j) {
      if (base + (int)j < n_plain) step(j, base + (int)j, kNo);
    });
  }
  // the masked tiles (the last few), one step each
  for (int it = n_plain; it < ntiles; ++it) {
    static_for<0, NBUF>([&](auto j) {
      if (it % NBUF == (int)j) step(j, it, kYes);
    });
  }
  // no load may still be landing in LDS when the workgroup ends
  wait_all();

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
  constexpr int QB = QATTN_QB;  // 32-query blocks per wave
  // dense: one workgroup of NW_DENSE waves per CU (NW_DENSE / 4 waves per
  // SIMD); sparse: one 128-row query block per 4-wave workgroup, two
  // workgroups per CU
  constexpr int NW_DENSE = QATTN_NW_DENSE;
  constexpr int WPE_DENSE = NW_DENSE / 4;
  constexpr int NW_SPARSE = 128 / (32 * QB);
  static_assert(NW_DENSE % 4 == 0, "whole waves per SIMD");
  if (sparse) {
    const dim3 grid(a.B * a.Hq * a.nqb);
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, QB, NW_SPARSE, 2, 3>), grid,
                       dim3(NW_SPARSE * 64), 0, stream, a);
  } else {
    const int rows_wg = 32 * QB * (NW_DENSE / a.g4);
    const int nrc = (a.N + rows_wg - 1) / rows_wg;
    const dim3 grid(a.B * a.Hkv * (a.group / a.g4) * nrc);
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, false, QB, NW_DENSE, WPE_DENSE, 3>),
                       grid, dim3(NW_DENSE * 64), 0, stream, a);
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
