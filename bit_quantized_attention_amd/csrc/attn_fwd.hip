// Quantized attention forward on gfx950 matrix cores.
//
// Work decomposition. A wave owns 32 query rows of one query head (one
// 32-column MFMA block). Dense: a workgroup of NW waves (8 at d = 128, 4 at
// d = 64) takes g4 = 4, 2 or 1 query heads of one kv head (the largest that
// divides the group size) times NW/g4 consecutive 32-row slabs, so all its
// waves share every K/V tile they stage (d = 128, GQA group 4: four heads x
// the same 64 rows). Sparse: a workgroup of
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
// Pipeline (one barrier per tile; each stage of K tile, its scale and V tile
// is one LDS object): the workgroups run the P V products of tile t-1
// inside the softmax of tile t, so each wave feeds its matrix unit while its
// vector unit works (dense d = 128: four stages; dense d = 64 and sparse:
// three, so that three or two workgroups fit a CU). The promoted and
// gathered variants run S, the softmax and P V of a tile in sequence (three
// stages) and the waves sharing a SIMD overlap each other's work. Q fragments stay in registers; every K
// tile carries its scale in a small tail of its stage (no scalar loads in
// the loop).
//
// Online softmax reference: a row's exponent reference m moves only when the
// tile's running max exceeds it by more than kTau (log2 units); otherwise P is
// taken against the stale reference (P <= 2^kTau) and the accumulator is not
// rescaled. The row max is only formed when a partial row sum says a move is
// possible; the move test is wave-uniform, so the common case costs neither
// the max nor the rescale.
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
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kKT = 64;             // keys per tile
constexpr float kTau = QATTN_SOFTMAX_REF_THRESHOLD;  // log2 units
// The INT8 product accumulates onto the bit pattern of 1.5 * 2^23: every
// |S| < 2^22 (d * 127^2 at most) then reads, as an fp32 number, exactly
// 1.5 * 2^23 + S, so no conversion instruction is needed.
constexpr int kSBias = 0x4B400000;
constexpr float kSBiasF = 12582912.0f;
// A lane's partial row sum above this (2^(kTau-1)) may hide an element past
// the reference by more than kTau; only then is the row max computed.
constexpr float kSumFilter = 128.0f;
constexpr int kMaxSparseTiles = 2048;
// longest gathered key list (64-key tiles of listed keys) per query block
constexpr int kMaxGatherKeys = 3072;

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
  // promoted path: the 16-bit Q and K and the K smoothing mean; head_hi
  // (adaptive precision) promotes every visible block of the flagged heads
  // and none of the others, in place of a kept list
  const uint16_t* q16;
  const uint16_t* k16;
  const float* k_mean;
  const int32_t* head_hi;
  // promoted path with an MX FP4 low path: E2M1 codes (two per byte) and E8M0
  // exponents (one per 32 channels) of the raw Q and the smoothed K
  const uint8_t* q4;
  const uint8_t* qe;
  const uint8_t* k4;
  const uint8_t* ke;
  // kv_idx / kv_cnt / max_keep hold key lists (gathered keys) instead of
  // block lists
  bool gather;
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
  // Promoted tiles: half a tile (32 keys) of the 16-bit K fills the same
  // KBUF bytes, in rows of 2*D bytes; the 16-bit product takes 16-deep
  // k-steps. Same swizzle rule as kswz for the longer rows.
  static constexpr int K16ROW = 2 * D;
  static constexpr int K16SLOTS = K16ROW / 16;
  static constexpr int KS16 = D / 16;
  static __device__ __forceinline__ int k16swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // MX FP4 low tiles: a K row is D/2 bytes of E2M1 codes (D/32 16-byte slots),
  // the 4-bit product takes 64-channel k-steps, and the row's D/32 exponent
  // bytes follow the tile in the tail. Swizzle: the 16 rows of a 16-lane read
  // phase (same slot) cover all 64 banks.
  static constexpr int K4ROW = D / 2;
  static constexpr int K4SLOTS = D / 32;
  static constexpr int K4BUF = kKT * K4ROW;
  static constexpr int KS4 = D / 64;
  static constexpr int K4EXP = D / 32;  // exponent bytes per key
  static __device__ __forceinline__ int k4swz(int r) { return D == 128 ? ((r >> 2) & 3) : ((r >> 3) & 1); }
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

template <int D, bool BF16, bool CAUSAL, bool SPARSE, int QB, int NW, int WPE, int NBUF, bool PROMOTE,
          bool GATHER, bool LOW4 = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_fwd_kernel(FwdArgs a) {
  using MM = Mma16<BF16>;
  using op_t = typename MM::op_t;
  using el_t = typename MM::el_t;
  using G = Geo<D>;
  constexpr int RW = 32 * QB;
  // lagged P V (the dense and the plain block-sparse layouts)
  constexpr bool kLAG = !PROMOTE && !GATHER;
  // promoted path: sparse layout (one 128-row query block per workgroup),
  // one 32-query block per wave
  static_assert(!PROMOTE || (SPARSE && QB == 1), "promoted path: sparse layout, QB = 1");
  // gathered keys: sparse layout; kv_idx holds key lists (max_keep entries per
  // query block) and a tile is 64 consecutive list entries
  static_assert(!GATHER || (SPARSE && QB == 1 && !PROMOTE), "gathered keys: sparse layout, QB = 1");
  // MX FP4 low tiles: only on the promoted path
  static_assert(!LOW4 || PROMOTE, "4-bit low tiles: promoted path");
  static_assert(!LOW4 || (G::K4BUF + kKT * G::K4EXP <= G::KBUF + 256), "4-bit K tile fits the K slot");
  constexpr int KPIECES = G::KBUF / 1024;  // 1 KB direct loads per K tile
  constexpr int VPIECES = G::VBUF / 1024;
  // Staging buffer j (K tile, the tail carrying its scale, V tile) is one
  // LDS object, always named with a compile-time index: the compiler can then
  // tell that an LDS read of one buffer does not depend on the DMA loads still
  // landing in another, and waits only for the loads of the buffer it reads.
  // (Its tracking has room for few objects; one per stage keeps every read of
  // the loop clear of the loads in flight.)
  static_assert(NBUF >= 3 && NBUF <= 6, "three to six staging buffers");
  constexpr int KB = G::KBUF + 256;  // K tile plus the tail carrying its scale
  constexpr int SB = KB + G::VBUF;   // one stage
  __shared__ __attribute__((aligned(16))) int8_t stage0[SB];
  __shared__ __attribute__((aligned(16))) int8_t stage1[SB];
  __shared__ __attribute__((aligned(16))) int8_t stage2[SB];
  __shared__ __attribute__((aligned(16))) int8_t stage3[NBUF > 3 ? SB : 16];
  __shared__ __attribute__((aligned(16))) int8_t stage4[NBUF > 4 ? SB : 16];
  __shared__ __attribute__((aligned(16))) int8_t stage5[NBUF > 5 ? SB : 16];
  auto stage = [&](auto i) -> int8_t* {
    constexpr int j = decltype(i)::value % NBUF;
    if constexpr (j == 0) return stage0;
    else if constexpr (j == 1) return stage1;
    else if constexpr (j == 2) return stage2;
    else if constexpr (j == 3) return stage3;
    else if constexpr (j == 4) return stage4;
    else return stage5;
  };
  auto kbuf = [&](auto i) -> int8_t* { return stage(i); };
  auto vbuf = [&](auto i) -> int8_t* { return stage(i) + KB; };
  __shared__ int16_t tile_list[SPARSE && !GATHER ? kMaxSparseTiles : 1];
  __shared__ __attribute__((aligned(16))) uint16_t key_list[GATHER ? kMaxGatherKeys : 1];
  // gathered tiles: each wave's fl32(alpha_q * k_scale) of the tile's 64 keys
  __shared__ __attribute__((aligned(16))) float key_alpha[GATHER ? NW * 64 : 1];
  __shared__ uint32_t kept_bits[PROMOTE ? kMaxSparseTiles / 32 : 1];
  __shared__ int n_list, n_list_plain, n_list_hi;

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
  int n_hi = 0;  // promoted tiles (each visited as two 32-key halves)
  if constexpr (PROMOTE) {
    // The kept list marks the promoted tiles in a bit set (so duplicates and
    // order do not matter); one ascending scan of the visible tiles then
    // writes the low tiles to tile_list[0, n1) and the promoted ones to
    // tile_list[n1, n1 + n_hi).
    const int nvis = CAUSAL ? min(a.nkb, wg_last_row / kKT + 1) : a.nkb;
    const int nwords = (nvis + 31) >> 5;
    const uint32_t fill = (a.head_hi != nullptr && a.head_hi[bhq] != 0) ? ~0u : 0u;
    for (int w = threadIdx.x; w < nwords; w += NW * 64) kept_bits[w] = fill;
    __syncthreads();
    if (a.head_hi == nullptr) {
      const int cnt = min(a.kv_cnt[bhq * a.nqb + qblk], min(a.max_keep, kMaxSparseTiles));
      const int32_t* src = a.kv_idx + (bhq * a.nqb + qblk) * a.max_keep;
      for (int e = threadIdx.x; e < cnt; e += NW * 64) {
        const int t = src[e];
        if (t >= 0 && t < nvis) atomicOr(&kept_bits[t >> 5], 1u << (t & 31));
      }
    }
    __syncthreads();
    if (wave == 0) {
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      auto is_kept = [&](int t) { return t < nvis && ((kept_bits[t >> 5] >> (t & 31)) & 1u) != 0u; };
      int nk = 0;
      for (int t0 = 0; t0 < nvis; t0 += 64) nk += __popcll(__ballot(is_kept(t0 + lane)));
      const int n1 = nvis - nk;
      int p1 = 0, p2 = 0, p1_plain = 0;
      for (int t0 = 0; t0 < nvis; t0 += 64) {
        const int t = t0 + lane;
        const bool kept = is_kept(t);
        const bool low = t < nvis && !kept;
        const uint64_t bl = __ballot(low);
        const uint64_t bk = __ballot(kept);
        if (low) tile_list[p1 + __popcll(bl & lt)] = (int16_t)t;
        if (kept) tile_list[n1 + p2 + __popcll(bk & lt)] = (int16_t)t;
        p1 += __popcll(bl);
        p2 += __popcll(bk);
        p1_plain += __popcll(__ballot(low && !masked(t)));
      }
      if (lane == 0) {
        n_list = n1;
        n_list_plain = p1_plain;
        n_list_hi = nk;
      }
    }
    __syncthreads();
    ntiles = n_list;
    n_plain = n_list_plain;
    n_hi = n_list_hi;
  } else if constexpr (GATHER) {
    // the key list (entries outside [0, N) or past the causal range dropped,
    // order kept); tiles are 64 consecutive entries. The unmasked tiles are
    // the whole tiles before the first entry past the workgroup's first row.
    if (wave == 0) {
      const int cap = min(a.max_keep, kMaxGatherKeys);
      const int32_t* src = a.kv_idx + (bhq * a.nqb + qblk) * a.max_keep;
      const int cnt = min(a.kv_cnt[bhq * a.nqb + qblk], cap);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int n = 0, first_late = INT_MAX;
      // eight 64-entry chunks per round, their loads all in flight together;
      // the first round reads up to the row's capacity without waiting for
      // the count (entries past it are masked below)
      int e0 = 0;
      do {
        int kc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = e0 + 64 * j + lane;
          kc[j] = e < cap ? src[e] : -1;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = kc[j];
          const bool ok = e0 + 64 * j + lane < cnt && k >= 0 && k < a.N &&
                          (!CAUSAL || k <= wg_last_row);
          const uint64_t bal = __ballot(ok);
          const int pos = n + __popcll(bal & lt);
          if (ok) key_list[pos] = (uint16_t)k;
          const uint64_t late = __ballot(ok && CAUSAL && k > wg_row0);
          if (late != 0ull && first_late == INT_MAX) {
            const int l0 = __builtin_ctzll(late);
            first_late = n + __popcll(bal & ((l0 == 0) ? 0ull : (~0ull >> (64 - l0))));
          }
          n += __popcll(bal);
        }
        e0 += 8 * 64;
      } while (e0 < cnt);
      if (lane == 0) {
        n_list = n;
        n_list_plain = min(first_late, n) / kKT;
      }
    }
    __syncthreads();
    ntiles = (n_list + kKT - 1) / kKT;
    n_plain = n_list_plain;
  } else if constexpr (SPARSE) {
    if (wave == 0) {
      const int cap = min(a.max_keep, kMaxSparseTiles);
      const int32_t* src = a.kv_idx + (bhq * a.nqb + qblk) * a.max_keep;
      // the first 64 entries are read together with the count (the row holds
      // max_keep entries) and serve both passes
      const int t_first = lane < cap ? src[lane] : -1;
      const int cnt = min(a.kv_cnt[bhq * a.nqb + qblk], cap);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int n = 0;
      for (int pass = 0; pass < 2; ++pass) {
        for (int e0 = 0; e0 < cnt; e0 += 64) {
          const int e = e0 + lane;
          const int t = e >= cnt ? -1 : e0 == 0 ? t_first : src[e];
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
    if constexpr (SPARSE && !GATHER) return tile_list[it];
    else return it;
  };
  // gathered keys: the key of list entry pos (entries past the list read its
  // last key, an empty list key 0: valid rows whose results are masked)
  const int n_keys = GATHER ? n_list : 0;
  auto listed_key = [&](int pos) -> int {
    if constexpr (GATHER) return n_keys > 0 ? (int)key_list[min(pos, n_keys - 1)] : 0;
    else return 0;
  };

  // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------------
  v4i qf[QB][G::KS];
  if (wave_live && !LOW4) {
    const int8_t* qg = a.q_i8 + (bhq * a.N + row0) * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const v4i*>(qg + (size_t)(32 * qb + l32) * D + 32 * ks + 16 * h);
  }
  const float alpha_q = (wave_live && !LOW4) ? a.q_scale[bhq * a.nqb + qblk] * a.c : 0.0f;
  const float* kscale = LOW4 ? nullptr : a.k_scale + (size_t)kvu * a.nkb;
  // 4-bit low tiles: the wave's query rows as MX FP4 B-operand fragments
  // (lane (l32, h): row row0 + l32, channels 64 ks + 32 h + [0, 32)) and
  // their exponents
  v4i q4f[LOW4 ? G::KS4 : 1];
  int q4e[LOW4 ? G::KS4 : 1];
  if constexpr (LOW4) {
    if (wave_live) {
      const size_t qr = bhq * a.N + row0 + l32;
#pragma unroll
      for (int ks = 0; ks < G::KS4; ++ks) {
        q4f[ks] = *reinterpret_cast<const v4i*>(a.q4 + qr * G::K4ROW + 32 * ks + 16 * h);
        q4e[ks] = a.qe[qr * G::K4EXP + 2 * ks + h];
      }
    }
  }

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
  auto load_k = [&](int t, int8_t* buf) {
    const int8_t* src = a.k_i8 + (kv_row0 + (size_t)t * kKT) * D;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int piece = (wave + NW * j) % KPIECES;
      lds_dma16(src + k_src_off(piece), buf + piece * 1024);
    }
  };
  // 4-bit K tile t: KPW loads per wave like an INT8 tile (pieces repeat when
  // the tile has fewer 1 KB pieces than the waves' loads; identical bytes)
  auto load_k4 = [&](int t, int8_t* buf) {
    constexpr int K4P = G::K4BUF / 1024;
    const int8_t* src = reinterpret_cast<const int8_t*>(a.k4) + (kv_row0 + (size_t)t * kKT) * G::K4ROW;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int piece = (wave + NW * j) % K4P;
      const int r = piece * (1024 / G::K4ROW) + lane / G::K4SLOTS;
      lds_dma16(src + r * G::K4ROW + (((lane % G::K4SLOTS) ^ G::k4swz(r)) * 16), buf + piece * 1024);
    }
  };
  // the tail word of a tile's stage: its K scale (INT8 tiles; all lanes the
  // same word), or (4-bit low path) its 64 keys' exponent bytes, lane l
  // bringing 4 of them (d = 64: 2 keys per word, lanes 32-63 repeat 0-31)
  auto tail_dma = [&](int t, int8_t* kb) {
    if constexpr (LOW4) {
      const int w = D == 128 ? lane : (lane & 31);
      lds_dma4(a.ke + (kv_row0 + (size_t)t * kKT) * G::K4EXP + 4 * w, kb + G::KBUF);
    } else {
      lds_dma4(kscale + t, kb + G::KBUF);
    }
  };
  auto tile_kscale = [&](const int8_t* buf) {
    return *reinterpret_cast<const float*>(buf + G::KBUF);
  };
  // gathered tile t: row r of the K and V tiles is listed key 64 t + r
  auto load_k_gather = [&](int t, int8_t* buf) {
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int piece = (wave + NW * j) % KPIECES;
      const int r = piece * (1024 / G::KROW) + lane / G::KSLOTS;
      const int key = listed_key(kKT * t + r);
      const int8_t* src = a.k_i8 + (kv_row0 + (size_t)key) * D +
                          (((lane % G::KSLOTS) ^ G::kswz(r)) * 16);
      lds_dma16(src, buf + piece * 1024);
    }
  };
  auto load_v_gather = [&](int t, int8_t* buf) {
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int piece = (wave + NW * j) % VPIECES;
      const int r = piece * (1024 / G::VROW) + lane / G::VSLOTS;
      const int key = listed_key(kKT * t + r);
      const int8_t* src = reinterpret_cast<const int8_t*>(a.v + (kv_row0 + (size_t)key) * D) +
                          (((lane % G::VSLOTS) ^ G::vswz(r)) * 16);
      lds_dma16(src, buf + piece * 1024);
    }
  };
  auto load_v = [&](int t, int8_t* buf) {
    const int8_t* src = reinterpret_cast<const int8_t*>(a.v + (kv_row0 + (size_t)t * kKT) * D);
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int piece = (wave + NW * j) % VPIECES;
      lds_dma16(src + v_src_off(piece), buf + piece * 1024);
    }
  };
  // Half hs of promoted tile t: its 32 rows of the 16-bit K, in the same
  // number of 1 KB loads as an INT8 K tile.
  auto k16_src_off = [&](int piece) -> uint32_t {
    const int r = piece * (1024 / G::K16ROW) + lane / G::K16SLOTS;
    return (uint32_t)(r * G::K16ROW + (((lane % G::K16SLOTS) ^ G::k16swz(r)) * 16));
  };
  auto load_k16 = [&](int t, int hs, int8_t* buf) {
    const int8_t* src = reinterpret_cast<const int8_t*>(a.k16 + (kv_row0 + (size_t)t * kKT + 32 * hs) * D);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int piece = (wave + NW * j) % KPIECES;
      lds_dma16(src + k16_src_off(piece), buf + piece * 1024);
    }
  };
  // Step vt of the whole sequence: INT8 tiles [0, ntiles), then (promoted
  // path) the two halves of each promoted tile. Steps past the end are
  // clamped to the last one, and an empty sequence (a kept list with no
  // usable entry) loads tile 0: such loads land in buffers nobody reads.
  const int nsteps = ntiles + 2 * n_hi;
  auto load_desc = [&](int vt, int& t, int& hs) {
    vt = min(vt, nsteps - 1);
    if (vt < 0) {
      t = 0;
      hs = -1;
      return;
    }
    if constexpr (PROMOTE) {
      if (vt < ntiles) {
        t = tile_list[vt];
        hs = -1;
      } else {
        const int u = vt - ntiles;
        t = tile_list[ntiles + (u >> 1)];
        hs = u & 1;
      }
    } else {
      t = tile_of(vt);
      hs = -1;
    }
  };
  // The K tile's scale rides along into the 256-byte tail of its buffer (all
  // 64 lanes load the same word), so the softmax reads it from LDS: no
  // scalar load, whose out-of-order return would make every LDS wait a full
  // wait. (A promoted half loads it too, unused, so that every step issues
  // the same number of loads.)
  auto issue = [&](int t, int hs, int8_t* kb, int8_t* vb) {
    if constexpr (GATHER) {
      // lane l brings the scale of row l's key into the tail
      load_k_gather(t, kb);
      lds_dma4(kscale + listed_key(kKT * t + lane) / kKT, kb + G::KBUF);
      load_v_gather(t, vb);
      return;
    }
    if constexpr (PROMOTE) {
      if (hs >= 0) load_k16(t, hs, kb);
      else if constexpr (LOW4) load_k4(t, kb);
      else load_k(t, kb);
    } else {
      load_k(t, kb);
    }
    tail_dma(t, kb);
    load_v(t, vb);
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
  // Initial accumulator of the S products: the bias pattern, held in
  // registers for the whole loop (the empty asm hides the constant, so it is
  // not rematerialized with 16 moves per tile).
  v16i sbias;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int bv = kSBias;
    asm volatile("" : "+v"(bv));
    sbias[r] = bv;
  }
  auto qk = [&](const int8_t* kbuf, v16i (&s)[2][QB]) {
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      v4i qv[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qv[qb] = qf[qb][ks];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v4i kf = *reinterpret_cast<const v4i*>(kbuf + kb * 32 * G::KROW + k_frag_off[ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (ks == 0) {
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qv[qb], sbias, 0, 0, 0);
          } else {
            s[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qv[qb], s[kb][qb], 0, 0, 0);
          }
        }
      }
    }
  };

  // softmax of one tile, one 32-query block at a time: S (as 1.5*2^23 + S in
  // fp32) -> P packed in the B-operand layout of the P V product, the lane's
  // partial row sum (fp32, of P before its 16-bit rounding) added to l.
  // With A = alpha * 1.5*2^23 split into A_hi + A_lo (exact), the fma
  // alpha*Sb - A_hi is alpha*S + A_lo, so the exponent alpha*S - m is
  // fma(alpha, Sb, -A_hi) - (m + A_lo): two roundings of numbers of the size
  // of the exponent itself. (One fma against a rounded A + m would shift a
  // tile's exponents by up to alpha/2, enough to flip the 16-bit rounding of
  // many P.)
  // The reference m follows the rule of the module comment, but the row max
  // is only formed when some lane's partial sum exceeds kSumFilter: a move
  // needs an element more than kTau above m, i.e. a P above 2^kTau. Then the
  // row max (an integer max3 tree) decides; rows that move get P again
  // against the new reference, and acc and l are rescaled (corr). With
  // MASKED (causal tiles reaching past the workgroup's first row), element
  // (kb, r), which holds key t*64 + 4h + off, is dropped when off > lim.
  // hook(qb, g) runs at the start of group g = 2*kb + half of the first pass
  // over query block qb (the lagged P V products of the previous tile
  // interleave there).
  auto softmax = [&](auto masked_c, const v16i (&s)[2][QB], float alpha, int t,
                     op_t (&pf)[2][QB][2], auto&& hook) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const float a_hi = alpha * kSBiasF;
    const float a_lo = __builtin_fmaf(alpha, kSBiasF, -a_hi);
    static_for<0, QB>([&](auto qbc) {
      constexpr int qb = decltype(qbc)::value;
      const int lim = (row0 + 32 * qb + l32) - (t * kKT + 4 * h);
      // P against reference m (-inf: every visible P is +inf, which forces
      // the row max below), and its partial sum
      auto exps = [&](float m, float ahi, auto&& grp_hook) -> float {
        const float cm = m + a_lo;
        // -0 is the additive identity, so the first additions fold away
        float lsum[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
        static_for<0, 4>([&](auto gc) {
          constexpr int kb = decltype(gc)::value >> 1;
          constexpr int half = decltype(gc)::value & 1;
          grp_hook(qbc, gc);
          {
            op_t pk;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * half + e;
              const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
              const float sb = __builtin_bit_cast(float, (int)s[kb][qb][r]);
              const float x = __builtin_fmaf(alpha, sb, -ahi) - cm;
              float pe = __builtin_amdgcn_exp2f(x);
              if constexpr (MASKED) pe = off > lim ? 0.0f : pe;
              lsum[e & 3] += pe;
              pk[e] = (el_t)pe;
            }
            pf[kb][qb][half] = pk;
          }
        });
        return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
      };
      float psum = exps(m_ref[qb], a_hi, hook);
      if (__ballot(psum > kSumFilter) != 0) {
        // row max over the lane's 32 keys (biased integers; masked keys
        // excluded), then over the other half-row
        int si[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            si[16 * kb + r] = (MASKED && off > lim) ? INT_MIN : (int)s[kb][qb][r];
          }
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
        // fl32(max S * alpha); -inf for a fully masked row, which never moves
        const float mx = mxi == INT_MIN ? -__builtin_inff() : (float)(mxi - kSBias) * alpha;
        const float m_old = m_ref[qb];
        const float mc = __builtin_fmaxf(m_old, mx);
        const bool move = mc > m_old + kTau;
        if (__ballot(move) != 0) {
          const float corr =
              move ? (m_old == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_old - mc)) : 1.0f;
          m_ref[qb] = move ? mc : m_old;
          // recompute from S (an opaque copy of a_hi keeps the compiler from
          // holding the 32 first-pass products live across the fast path)
          float ahi = a_hi;
          asm volatile("" : "+v"(ahi));
          psum = exps(m_ref[qb], ahi, [](auto, auto) {});
          l_run[qb] *= corr;
#pragma unroll
          for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][qb][r] *= corr;
        }
      }
      l_run[qb] += psum;
    });
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
  // The V^T fragments of one 16-key group g = 2*kb + half (one per channel
  // block db)
  auto load_vgrp = [&](const int8_t* vbuf, int g, op_t (&vf)[G::DB]) {
    const int kb = g >> 1, half = g & 1;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
      const int8_t* p = vbuf + (kb * 32 + 16 * half) * G::VROW + v_frag_off[db];
      const v4s lo = lds_read_tr16(p);
      const v4s hi = lds_read_tr16(p + 8 * G::VROW);
      const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      vf[db] = __builtin_bit_cast(op_t, both);
    }
  };
  // P V over the tile's four 16-key groups, the fragments of the group after
  // next in flight while a group's products run (two fragment sets; the
  // scheduling barriers keep the compiler from sinking the reads next to
  // their use, which would expose the LDS latency at every product). Channel
  // blocks innermost: consecutive matrix instructions update different
  // accumulators, so none waits for the one before it.
  auto pv = [&](const int8_t* vbuf, const op_t (&pf)[2][QB][2]) {
    op_t va[G::DB], vb[G::DB];
    load_vgrp(vbuf, 0, va);
    load_vgrp(vbuf, 1, vb);
    static_for<0, 4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      op_t (&vf)[G::DB] = (g & 1) ? vb : va;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[db][qb] = MM::mma(vf[db], pf[g >> 1][qb][g & 1], acc[db][qb]);
      if constexpr (g + 2 < 4) load_vgrp(vbuf, g + 2, vf);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- promoted halves (32 keys of a promoted tile, 16-bit Q K^T) -----------------
  // S^T = K16 . Q16^T on v_mfma_f32_32x32x16_{bf16,f16}: lane (l32, h) holds
  // channels 16*ks + 8*h + [0, 8) of K row l32 (A) and of its query row (B),
  // the same lane layout as the INT8 product with 16-deep k-steps, so the fp32
  // result has the S^T layout the softmax and P V already use.
  int k16_frag_off[PROMOTE ? G::KS16 : 1];
  if constexpr (PROMOTE) {
#pragma unroll
    for (int ks = 0; ks < G::KS16; ++ks)
      k16_frag_off[ks] = l32 * G::K16ROW + (((2 * ks + h) ^ G::k16swz(l32)) * 16);
  }
  auto qk16 = [&](const int8_t* kb, const op_t (&qf16)[G::KS16], v16f& s) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < G::KS16; ++ks) {
      const op_t kf = *reinterpret_cast<const op_t*>(kb + k16_frag_off[ks]);
      if (ks == 0) {
        v16f z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
        s = MM::mma(kf, qf16[0], z);
      } else {
        s = MM::mma(kf, qf16[ks], s);
      }
    }
  };
  // Online softmax over a half: the logit of element r is c*S - cq, cq =
  // fl32(c * (q . k_mean)) (the smoothing's per-row constant, which puts these
  // logits in the INT8 path's frame), so the exponent is fma(c, S, -(cq + m)).
  // Same reference rule, filter and rescale as the INT8 softmax; element r
  // holds key key0 + 8*(r/4) + 4*h + r%4 and P goes out as the two 16-key
  // groups of this 32-key block.
  auto softmax_hi = [&](const v16f& s, int key0, float cq, op_t (&pf)[2]) __attribute__((always_inline)) {
    const int lim = (row0 + l32) - (key0 + 4 * h);
    auto exps = [&](float m) -> float {
      const float cm = cq + m;
      float lsum[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        op_t pk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hf + e;
          const int off = 8 * (r >> 2) + (r & 3);
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(a.c, s[r], -cm));
          if constexpr (CAUSAL) pe = off > lim ? 0.0f : pe;
          lsum[e & 3] += pe;
          pk[e] = (el_t)pe;
        }
        pf[hf] = pk;
      }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    float psum = exps(m_ref[0]);
    if (__ballot(psum > kSumFilter) != 0) {
      float mxs = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        mxs = __builtin_fmaxf(mxs, (CAUSAL && off > lim) ? -__builtin_inff() : s[r]);
      }
      {
        const int mi = __builtin_bit_cast(int, mxs);
        const auto sw = __builtin_amdgcn_permlane32_swap(mi, mi, false, false);
        mxs = __builtin_fmaxf(__builtin_bit_cast(float, (int)sw[0]), __builtin_bit_cast(float, (int)sw[1]));
      }
      // c > 0: the max logit is the logit of the max product (-inf when the
      // row sees no key of this half)
      const float mx = __builtin_fmaf(a.c, mxs, -cq);
      const float m_old = m_ref[0];
      const float mc = __builtin_fmaxf(m_old, mx);
      const bool move = mc > m_old + kTau;
      if (__ballot(move) != 0) {
        const float corr =
            move ? (m_old == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_old - mc)) : 1.0f;
        m_ref[0] = move ? mc : m_old;
        psum = exps(m_ref[0]);
        l_run[0] *= corr;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][0][r] *= corr;
      }
    }
    l_run[0] += psum;
  };
  // P V of a half: the two 16-key groups of 32-key block hs of the staged V
  // tile (hs dispatched to compile-time offsets: with a runtime offset the
  // compiler cannot tell the reads from the loads landing in other buffers
  // and waits for all of them)
  auto pv_hi = [&](const int8_t* vb, int hs, const op_t (&pf)[2]) __attribute__((always_inline)) {
    static_for<0, 2>([&](auto hc) {
      constexpr int H = decltype(hc)::value;
      if (hs == H) {
        op_t va[G::DB], vc[G::DB];
        load_vgrp(vb, 2 * H, va);
        load_vgrp(vb, 2 * H + 1, vc);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[db][0] = MM::mma(va[db], pf[0], acc[db][0]);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[db][0] = MM::mma(vc[db], pf[1], acc[db][0]);
      }
    });
  };

  // ---- 4-bit low tiles (MX FP4 Q K^T, the promoted path's low path) -----------
  // S^T = K4 . Q4^T on v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands and
  // E8M0 scales per 32 channels (lane (l32, h): key row 32 kb + l32 and query
  // row l32, channels 64 ks + 32 h + [0, 32)); the fp32 result has the S^T
  // layout of the INT8 product. The products of E2M1 values are exact, and so
  // is their fp32 sum unless the summed groups' exponents span more than about
  // ten binades.
  auto qk4 = [&](const int8_t* kbp, v16f (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = 32 * kb + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < G::KS4; ++ks) {
        const v4i kf = *reinterpret_cast<const v4i*>(kbp + r * G::K4ROW + (((2 * ks + h) ^ G::k4swz(r)) * 16));
        const int ke = (int)*reinterpret_cast<const uint8_t*>(kbp + G::KBUF + r * G::K4EXP + 2 * ks + h);
        const v8i ka = {kf[0], kf[1], kf[2], kf[3], 0, 0, 0, 0};
        const v8i qa = {q4f[ks][0], q4f[ks][1], q4f[ks][2], q4f[ks][3], 0, 0, 0, 0};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa, s[kb], 4, 4, 0, ke, 0, q4e[ks]);
      }
    }
  };
  // Online softmax of a 4-bit tile: the logit of element (kb, r) is
  // c * S (the smoothed keys put it in the INT8 path's frame), so the
  // exponent is one fma, fma(c, S, -m). Element (kb, r) holds key
  // t*64 + 32 kb + 8 (r/4) + 4 h + r%4. Reference rule, filter and rescale as
  // in softmax.
  auto softmax_f = [&](auto masked_c, const v16f (&s)[2], int t, op_t (&pf)[2][QB][2]) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int lim = (row0 + l32) - (t * kKT + 4 * h);
    auto exps = [&](float m) -> float {
      float lsum[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          op_t pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * hf + e;
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(a.c, s[kb][r], -m));
            if constexpr (MASKED) pe = off > lim ? 0.0f : pe;
            lsum[e & 3] += pe;
            pk[e] = (el_t)pe;
          }
          pf[kb][0][hf] = pk;
        }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    float psum = exps(m_ref[0]);
    if (__ballot(psum > kSumFilter) != 0) {
      float mxs = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          mxs = __builtin_fmaxf(mxs, (MASKED && off > lim) ? -__builtin_inff() : s[kb][r]);
        }
      {
        const int mi = __builtin_bit_cast(int, mxs);
        const auto sw = __builtin_amdgcn_permlane32_swap(mi, mi, false, false);
        mxs = __builtin_fmaxf(__builtin_bit_cast(float, (int)sw[0]), __builtin_bit_cast(float, (int)sw[1]));
      }
      // c > 0: the max logit is the logit of the max product (-inf when the
      // row sees no key of this tile)
      const float mx = a.c * mxs;
      const float m_old = m_ref[0];
      const float mc = __builtin_fmaxf(m_old, mx);
      const bool move = mc > m_old + kTau;
      if (__ballot(move) != 0) {
        const float corr =
            move ? (m_old == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_old - mc)) : 1.0f;
        m_ref[0] = move ? mc : m_old;
        psum = exps(m_ref[0]);
        l_run[0] *= corr;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][0][r] *= corr;
      }
    }
    l_run[0] += psum;
  };

  // ---- gathered tiles: a scale per key ----------------------------------------
  // Element (kb, r) of the lane's 32 keys is row kb*32 + 8*(r/4) + 4*h + r%4
  // of the tile, i.e. list entry 64*it + that row. Its logit is
  // fl32(S * fl32(alpha_q * sk)) with sk the row's scale from the tile tail;
  // P = exp2(fl32(logit - m)). Masked tiles drop entries past the list and,
  // under causal masking, keys past the row. Reference rule, filter and rescale as in softmax.
  auto softmax_gather = [&](auto masked_c, const v16i (&s)[2][QB], const int8_t* kb_buf, int it,
                            op_t (&pf)[2][QB][2]) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const float* tail = reinterpret_cast<const float*>(kb_buf + G::KBUF);
    const int row = row0 + l32;
    // lane l forms key l's alpha once for the wave (its own LDS slot: the
    // wave's reads below see its write)
    float* wal = key_alpha + wave * 64;
    wal[lane] = alpha_q * tail[lane];
    float x[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int rr = kb * 32 + 8 * g4 + 4 * h;  // first of the 4 rows
        const float4 al4 = *reinterpret_cast<const float4*>(wal + rr);
        const float alv[4] = {al4.x, al4.y, al4.z, al4.w};
        int keyv[4] = {0, 0, 0, 0};
        if constexpr (MASKED) {
          const uint2 kw = *reinterpret_cast<const uint2*>(&key_list[kKT * it + rr]);
          keyv[0] = (int)(kw.x & 0xffffu);
          keyv[1] = (int)(kw.x >> 16);
          keyv[2] = (int)(kw.y & 0xffffu);
          keyv[3] = (int)(kw.y >> 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          const float S = __builtin_bit_cast(float, (int)s[kb][0][r]) - kSBiasF;  // exact
          const float alpha = alv[e];
          float v = S * alpha;
          if constexpr (MASKED) {
            if (kKT * it + rr + e >= n_keys || (CAUSAL && keyv[e] > row)) v = -__builtin_inff();
          }
          x[kb][r] = v;
        }
      }
    auto exps = [&](float m) -> float {
      float lsum[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          op_t pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float pe = __builtin_amdgcn_exp2f(x[kb][8 * hf + e] - m);
            // a dropped element gives 0 also while m is still -inf (where
            // -inf - m would give NaN), as in the block softmax
            if constexpr (MASKED) pe = x[kb][8 * hf + e] == -__builtin_inff() ? 0.0f : pe;
            lsum[e & 3] += pe;
            pk[e] = (el_t)pe;
          }
          pf[kb][0][hf] = pk;
        }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    float psum = exps(m_ref[0]);
    if (__ballot(psum > kSumFilter) != 0) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, x[kb][r]);
      {
        const int mi = __builtin_bit_cast(int, mx);
        const auto sw = __builtin_amdgcn_permlane32_swap(mi, mi, false, false);
        mx = __builtin_fmaxf(__builtin_bit_cast(float, (int)sw[0]), __builtin_bit_cast(float, (int)sw[1]));
      }
      const float m_old = m_ref[0];
      const float mc = __builtin_fmaxf(m_old, mx);
      const bool move = mc > m_old + kTau;
      if (__ballot(move) != 0) {
        const float corr =
            move ? (m_old == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_old - mc)) : 1.0f;
        m_ref[0] = move ? mc : m_old;
        psum = exps(m_ref[0]);
        l_run[0] *= corr;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][0][r] *= corr;
      }
    }
    l_run[0] += psum;
  };

  // ---- pipeline ---------------------------------------------------------------------
  // Tile j's K (with its scale) and V live in buffer j % NBUF. Iteration it
  // issues the loads of tile it+PD into buffer (it+PD) % NBUF, whose last
  // readers ran before the previous barrier, computes S = K Q^T and the
  // softmax of tile it, then waits until only the loads of the last PD-1
  // iterations are in flight (tile it+1 has landed) and passes the barrier.
  // Tiles past the end are clamped to the last tile (never read), so each
  // iteration issues the same loads. The loops are unrolled NBUF times so
  // that every buffer is named at compile time.
  //
  // Lagged P V: iteration it runs the P V products of tile it-1 inside the
  // softmax of tile it, four matrix instructions per 16-key group of
  // exponentials, so each wave keeps its matrix unit busy while its vector
  // unit works (P of consecutive tiles alternates between two register sets;
  // the first iteration multiplies a copy of tile 0's V by a zero P).
  // V(it-1) is still read in iteration it, so the prefetch distance is
  // NBUF-2: two tiles in the d = 128 dense layout (four stages), one in the
  // d = 64 dense and the block-sparse layouts, whose three stages keep three
  // or two workgroups per CU (four stages and one workgroup measured
  // slower). With an odd NBUF the loops are unrolled 2 NBUF times, so that
  // P's register set stays a compile-time choice. Otherwise
  // (promoted, gathered) each wave runs S, the softmax and P V of a tile in
  // sequence and the waves sharing a SIMD overlap each other's work.
  static_assert(!kLAG || NBUF == 3 || NBUF == 4 || NBUF == 6, "lagged products: three, four or six stages");
  constexpr int UNR = (kLAG && (NBUF & 1)) ? 2 * NBUF : NBUF;
  // prefetch distance (tiles) and the furthest tile the next iteration reads
  constexpr int PD = kLAG ? NBUF - 2 : NBUF - 1;
  static_for<0, PD>([&](auto j) {
    int tt, hs;
    load_desc((int)j, tt, hs);
    issue(tt, hs, kbuf(j), vbuf(j));
  });
  // lagged: the first iteration's "previous" V buffer gets tile 0's V too, so
  // that its zero P meets finite values (and the buffer is named at compile
  // time: a runtime choice of LDS buffer makes the compiler wait for every
  // load in flight before reading it); an empty kept list reads tile 0
  if constexpr (kLAG) load_v(ntiles > 0 ? tile_of(0) : 0, vbuf(std::integral_constant<int, NBUF - 1>{}));
  wait_all();
  __syncthreads();

  constexpr int kLoadsPerIt = KPW + 1 + VPW;  // K pieces, the K scale, V pieces
  constexpr auto vmcnt = [](int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); };
  static_assert((PD - 1) * kLoadsPerIt < 64, "vmcnt range");
  constexpr std::integral_constant<bool, true> kYes{};
  constexpr std::integral_constant<bool, false> kNo{};

  // lagged: P of even / odd tiles; the "previous" P of the first tile is zero
  op_t p_even[2][QB][2], p_odd[2][QB][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) p_odd[kb][qb][hf][e] = (el_t)0.0f;
  auto step = [&](auto jc, int it, auto masked_c) {
    constexpr int J = decltype(jc)::value;
    const std::integral_constant<int, J % NBUF> cur{};
    const std::integral_constant<int, (J + PD) % NBUF> nxt{};
    const std::integral_constant<int, (J + NBUF - 1) % NBUF> prv{};
    int tl, tl_hs;
    load_desc(it + PD, tl, tl_hs);
    // Every wave issues the loads at the same place, live or not, after the
    // reads of the current K tile: a separate branch for waves without rows
    // would merge its freshly issued loads into the live path's wait state.
    const int t = tile_of(it);
    v16i s[2][QB];
    float alpha = 0.0f;
    if constexpr (kLAG) {
      // (NBUF is even or the loops run 2 NBUF steps, so J and it have the
      // same parity)
      const op_t (&p_in)[2][QB][2] = (J & 1) ? p_even : p_odd;
      op_t (&p_out)[2][QB][2] = (J & 1) ? p_odd : p_even;
      const int8_t* vp = vbuf(prv);
      // QB = 1: two fragment sets, refilled two groups ahead; QB > 1: all
      // four groups of V(t-1) at once, each set shared by the QB blocks
      constexpr int NVS = QB == 1 ? 2 : 4;
      op_t vset[NVS][G::DB];
      // QB = 1: the second 32-key block's INT8 products (kb = 1) run inside
      // the first two softmax groups, which only read the first block's S:
      // the matrix unit then has work while the softmax starts, instead of a
      // phase of products with the vector unit idle (d = 64: one product per
      // group, 0.9 % faster in the three-workgroup layout)
      constexpr bool kSplitQK = QB == 1;
      v4i kf1[G::KS];
      if (wave_live) {
        alpha = alpha_q * tile_kscale(kbuf(cur));
        static_for<0, NVS>([&](auto gc) { load_vgrp(vp, decltype(gc)::value, vset[decltype(gc)::value]); });
        if constexpr (kSplitQK) {
          const int8_t* kbp = kbuf(cur);
#pragma unroll
          for (int ks = 0; ks < G::KS; ++ks)
            kf1[ks] = *reinterpret_cast<const v4i*>(kbp + 32 * G::KROW + k_frag_off[ks]);
#pragma unroll
          for (int ks = 0; ks < G::KS; ++ks) {
            const v4i kf = *reinterpret_cast<const v4i*>(kbp + k_frag_off[ks]);
            s[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[0][ks], ks == 0 ? sbias : s[0][0], 0, 0, 0);
          }
        } else {
          qk(kbuf(cur), s);
        }
      }
      issue(tl, tl_hs, kbuf(nxt), vbuf(nxt));
      if (wave_live) {
        auto lagged_pv = [&](auto qbc, auto gc) {
          constexpr int qb = decltype(qbc)::value;
          constexpr int g = decltype(gc)::value;
          // each group's products stay at the start of its own 16-key group
          // of exponentials: left free, the compiler hoists all of them to
          // the top of the tile and the second half of the softmax runs with
          // the matrix unit idle (1.5 % at d = 64, 0.5 % at d = 128)
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kSplitQK && g < 2) {
            // k-steps [g*KS/2, (g+1)*KS/2) of the kb = 1 product
#pragma unroll
            for (int ks = g * G::KS / 2; ks < (g + 1) * G::KS / 2; ++ks)
              s[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf1[ks], qf[0][ks], ks == 0 ? sbias : s[1][0],
                                                              0, 0, 0);
          }
          op_t (&vf)[G::DB] = vset[g % NVS];
#pragma unroll
          for (int db = 0; db < G::DB; ++db)
            acc[db][qb] = MM::mma(vf[db], p_in[g >> 1][qb][g & 1], acc[db][qb]);
          if constexpr (QB == 1 && g + 2 < 4) load_vgrp(vp, g + 2, vf);
        };
        softmax(masked_c, s, alpha, t, p_out, lagged_pv);
      }
    } else if constexpr (LOW4) {
      v16f s4[2];
      if (wave_live) qk4(kbuf(cur), s4);
      issue(tl, tl_hs, kbuf(nxt), vbuf(nxt));
      if (wave_live) {
        op_t p[2][QB][2];
        softmax_f(masked_c, s4, t, p);
        pv(vbuf(cur), p);
      }
    } else {
      if (wave_live) {
        if constexpr (!GATHER) alpha = alpha_q * tile_kscale(kbuf(cur));
        qk(kbuf(cur), s);
      }
      issue(tl, tl_hs, kbuf(nxt), vbuf(nxt));
      if (wave_live) {
        op_t p[2][QB][2];
        if constexpr (GATHER) softmax_gather(masked_c, s, kbuf(cur), it, p);
        else softmax(masked_c, s, alpha, t, p, [](auto, auto) {});
        pv(vbuf(cur), p);
      }
    }
    // The masked steps (a few per workgroup) wait for every load: any memory
    // instruction the compiler adds there is then covered too.
    if constexpr (decltype(masked_c)::value) {
      wait_all();
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt((PD - 1) * kLoadsPerIt));
    }
    barrier();
  };
  for (int base = 0; base < n_plain; base += UNR) {
    static_for<0, UNR>([&](auto j) {
      if (base + (int)j < n_plain) step(j, base + (int)j, kNo);
    });
  }
  // the masked tiles (the last few), one step each
  for (int it = n_plain; it < ntiles; ++it) {
    static_for<0, UNR>([&](auto j) {
      if (it % UNR == (int)j) step(j, it, kYes);
    });
  }
  // promoted path: the halves of the promoted tiles, after the INT8 tiles
  // (whose last steps have already prefetched the first halves)
  if constexpr (PROMOTE) {
    if (n_hi > 0) {
      // the wave's 16-bit query row fragments and q . k_mean (fp32; the two
      // lane halves hold the two halves of the row's channels)
      op_t qf16[G::KS16];
      const uint16_t* qg = a.q16 + (bhq * a.N + row0 + l32) * D;
      const float* mean = a.k_mean + (size_t)kvu * D;
      float part = 0.0f;
#pragma unroll
      for (int ks = 0; ks < G::KS16; ++ks) {
        qf16[ks] = *reinterpret_cast<const op_t*>(qg + 16 * ks + 8 * h);
        const float4 m0 = *reinterpret_cast<const float4*>(mean + 16 * ks + 8 * h);
        const float4 m1 = *reinterpret_cast<const float4*>(mean + 16 * ks + 8 * h + 4);
        const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)qf16[ks][e], mv[e], part);
      }
      const float cq = a.c * (part + __shfl_xor(part, 32, 64));
      auto step_hi = [&](auto jc, int it) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        const std::integral_constant<int, J % NBUF> cur{};
        const std::integral_constant<int, (J + PD) % NBUF> nxt{};
        // the step PD ahead is a promoted half too (clamped to the last)
        const int ul = min(it + PD, nsteps - 1) - ntiles;
        const int tl = tile_list[ntiles + (ul >> 1)];
        const int u = it - ntiles;
        const int t = tile_list[ntiles + (u >> 1)];
        const int hs = u & 1;
        v16f s;
        qk16(kbuf(cur), qf16, s);
        load_k16(tl, ul & 1, kbuf(nxt));
        tail_dma(tl, kbuf(nxt));
        load_v(tl, vbuf(nxt));
        op_t p[2];
        softmax_hi(s, t * kKT + 32 * hs, cq, p);
        pv_hi(vbuf(cur), hs, p);
        __builtin_amdgcn_s_waitcnt(vmcnt((PD - 1) * kLoadsPerIt));
        barrier();
      };
      // unrolled NBUF times from the stage the first half lands in, so that
      // consecutive steps name their buffers at compile time (a dispatch per
      // step would merge the wait states of all buffers at the loop head)
      auto hi_group = [&](auto j0c) __attribute__((always_inline)) {
        constexpr int J0 = decltype(j0c)::value;
        for (int base = ntiles; base + NBUF <= nsteps; base += NBUF) {
          static_for<0, NBUF>([&](auto j) {
            step_hi(std::integral_constant<int, (J0 + decltype(j)::value) % NBUF>{}, base + (int)j);
          });
        }
      };
      static_for<0, NBUF>([&](auto j0) {
        if (ntiles % NBUF == (int)j0) hi_group(j0);
      });
      for (int it = nsteps - (nsteps - ntiles) % NBUF; it < nsteps; ++it) {
        static_for<0, NBUF>([&](auto j) {
          if (it % NBUF == (int)j) step_hi(j, it);
        });
      }
    }
  }
  // no load may still be landing in LDS when the workgroup ends
  wait_all();
  if constexpr (kLAG) {
    // the last tile's P V (its buffer has landed and is not reloaded)
    if (wave_live && ntiles > 0) {
      static_for<0, UNR>([&](auto j) {
        if ((ntiles - 1) % UNR == (int)j) pv(vbuf(j), (j & 1) ? p_odd : p_even);
      });
    }
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

#ifndef QATTN_NW_DENSE64
#define QATTN_NW_DENSE64 4
#endif
#ifndef QATTN_WPE_DENSE_SMALL
#define QATTN_WPE_DENSE_SMALL 3
#endif
#ifndef QATTN_NW_DENSE
#define QATTN_NW_DENSE 8
#endif
#ifndef QATTN_QB
#define QATTN_QB 1
#endif
#ifndef QATTN_QB_DENSE
#define QATTN_QB_DENSE 1
#endif

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_dc(const FwdArgs& a, bool sparse, hipStream_t stream) {
  constexpr int QB = QATTN_QB;     // 32-query blocks per wave (sparse)
  constexpr int QBD = QATTN_QB_DENSE;  // 32-query blocks per wave (dense)
  // dense, d = 128: one 8-wave workgroup per CU (two waves per SIMD sharing
  // each staged tile); dense, d = 64: three 4-wave workgroups per CU, so that
  // the three waves on a SIMD pass independent barriers and one wave's
  // softmax overlaps another's products (5 % faster than one 8-wave
  // workgroup at the 4K non-causal d = 64 workload; the same split at
  // d = 128 was 1.3 % slower); sparse: one 128-row query block per 4-wave
  // workgroup, two workgroups per CU
  constexpr int NW_DENSE = (D == 64 ? QATTN_NW_DENSE64 : QATTN_NW_DENSE) / QBD;
  constexpr int WPE_DENSE = NW_DENSE >= 8 ? NW_DENSE / 4 : QATTN_WPE_DENSE_SMALL;
  constexpr int NW_SPARSE = 128 / (32 * QB);
  static_assert(NW_DENSE % 4 == 0, "whole waves per SIMD");
  if (sparse) {
    const dim3 grid(a.B * a.Hq * a.nqb);
    if (a.gather) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, 1, 4, 2, 3, false, true>), grid,
                         dim3(4 * 64), 0, stream, a);
    } else if (a.q16 != nullptr && a.k4 != nullptr) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, 1, 4, 2, 3, true, false, true>), grid,
                         dim3(4 * 64), 0, stream, a);
    } else if (a.q16 != nullptr) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, 1, 4, 2, 3, true, false>), grid,
                         dim3(4 * 64), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, true, QB, NW_SPARSE, 2, 3, false, false>),
                         grid, dim3(NW_SPARSE * 64), 0, stream, a);
    }
  } else {
    const int rows_wg = 32 * QBD * (NW_DENSE / a.g4);
    const int nrc = (a.N + rows_wg - 1) / rows_wg;
    const dim3 grid(a.B * a.Hkv * (a.group / a.g4) * nrc);
    constexpr int NBUF_DENSE = NW_DENSE * QBD >= 8 ? 4 : 3;
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, CAUSAL, false, QBD, NW_DENSE, WPE_DENSE, NBUF_DENSE, false,
                                        false>),
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
int fwd_max_gather_keys() { return kMaxGatherKeys; }

hipError_t launch_attn_fwd(const Shape& s, const int8_t* q_i8, const float* q_scale,
                           const int8_t* k_i8, const float* k_scale, const void* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, int max_keep,
                           const void* q16, const void* k16, const float* k_mean,
                           const int32_t* head_hi, bool gather, void* o, float* lse,
                           hipStream_t stream, const Fp4Codes* low4) {
  FwdArgs a;
  a.q4 = low4 ? low4->q4 : nullptr;
  a.qe = low4 ? low4->qe : nullptr;
  a.k4 = low4 ? low4->k4 : nullptr;
  a.ke = low4 ? low4->ke : nullptr;
  a.q_i8 = q_i8;
  a.q_scale = q_scale;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.q16 = static_cast<const uint16_t*>(q16);
  a.k16 = static_cast<const uint16_t*>(k16);
  a.k_mean = k_mean;
  a.head_hi = head_hi;
  a.gather = gather;
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
  const bool sparse = kv_idx != nullptr || head_hi != nullptr;
  if (s.d == 128)
    return s.bf16 ? launch_d<128, true>(a, s.causal, sparse, stream)
                  : launch_d<128, false>(a, s.causal, sparse, stream);
  return s.bf16 ? launch_d<64, true>(a, s.causal, sparse, stream)
                : launch_d<64, false>(a, s.causal, sparse, stream);
}

}  // namespace qattn
