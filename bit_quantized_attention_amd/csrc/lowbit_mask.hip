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
//      estimate. The key blocks the four waves share come through a ring of
//      four LDS stages filled by direct global-to-LDS loads (each wave brings
//      a quarter, three blocks ahead); the block maxima are software-
//      pipelined against the products (see the loop).
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

// Integer key with the order of the float values (every value but NaN): the
// magnitude bits of negative values are flipped. The map is its own inverse.
__device__ __forceinline__ int order_key(float v) {
  const int x = __float_as_int(v);
  return x ^ ((x >> 31) & 0x7fffffff);
}

// Max over the 64 lanes without LDS round trips (a shuffle chain waits for
// each of its six LDS permutes): DPP butterflies within each row of 16 lanes
// (xor 1 and xor 2 by quad permutes, then the half-row and row mirrors), then
// the row broadcasts of lanes 15 and 31 fold the four rows upward. Lane 63
// ends with the maximum over all lanes. On integer keys, with INT_MIN for the
// lanes a broadcast leaves out, each step is one DPP max instruction.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_max_key(int v) {
  return max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ int wave_max_key_to_lane63(int v) {
  v = dpp_max_key<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_key<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_key<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_key<0x140, 0xF>(v);  // row_mirror: every lane holds its row's max
  v = dpp_max_key<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_key<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Raw buffer over `bytes` bytes at p (offsets in bytes, no stride; loads past
// the end return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// One FP4 x FP4 product step: the key operand's E8M0 scale is byte 0 of ke,
// the query operand's byte SEL of qe (every lane's qe holds its row's
// scales, shifted so that byte 2 ks is the one for its 32 channels of k-step
// ks).
template <int SEL>
__device__ __forceinline__ v16f mfma_fp4(v8i k, v8i q, v16f c, int ke, int qe) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k, q, c, 4, 4, 0, ke, SEL, qe);
}

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct ScoreArgs {
  LowbitLayout L;
  int B, Hq, Hkv, group, N, nqb, nkb, causal;
};

// 16 or 4 bytes per lane from global memory straight into LDS at
// lds_base + size * lane (global_load_lds; the LDS base goes to M0)
template <int SIZE>
__device__ __forceinline__ void lds_dma(const void* g, uint8_t* lds_base) {
  static_assert(SIZE == 16 || SIZE == 4, "dword or 16-byte pieces");
  const auto src = (const void __attribute__((address_space(1)))*)g;
  const auto dst = (void __attribute__((address_space(3)))*)lds_base;
  if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// s_waitcnt immediate (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

template <int D>
__global__ __launch_bounds__(256) void lowbit_score_kernel(ScoreArgs a) {
  constexpr int KS = D / 64;      // 64-channel k-steps of the FP4 product
  constexpr int RB = 4;           // 32-row blocks of a 128-row query block
  constexpr int ROWB = D / 2;     // code bytes per key
  constexpr int ROWE = D / kMx;   // scale bytes per key (4 or 2)
  // LDS ring of key blocks: a block's codes (64 rows, 16-byte slots
  // XOR-swizzled by row so that the 16 rows of a 16-lane read phase cover
  // all 64 banks), then its scales
  constexpr int NST = 4;
  constexpr int CODEB = kKBlock * ROWB;
  constexpr int STAGE = CODEB + 256;  // the scales: 64 x ROWE bytes in 256
  constexpr int NPIECE = CODEB / 1024;  // 1 KB DMA pieces per block
  constexpr int SLOTS = ROWB / 16;
  // One LDS object per stage, always named with a compile-time index: the
  // compiler then knows that a read of one stage does not wait for the DMA
  // still landing in the others.
  __shared__ __attribute__((aligned(16))) uint8_t ring0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[STAGE];
  auto stage = [&](auto st_c) -> uint8_t* {
    constexpr int st = decltype(st_c)::value % NST;
    if constexpr (st == 0) return ring0;
    else if constexpr (st == 1) return ring1;
    else if constexpr (st == 2) return ring2;
    else return ring3;
  };
  auto swz = [](int r) { return D == 128 ? ((r >> 2) & 3) : ((r >> 3) & 1); };

  const int lane = threadIdx.x & 63;
  // wave index as a uniform (scalar) value: the wave's query head and its
  // addresses stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  // longest causal rows first
  const int slot = blockIdx.x % (a.B * a.Hkv);
  const int rank = blockIdx.x / (a.B * a.Hkv);
  const int i = a.causal ? a.nqb - 1 - rank : rank;
  const int b = slot / a.Hkv;
  const int hk = slot % a.Hkv;
  const int nvalid = a.causal ? min(a.nkb, (kQBlock * i + kQBlock - 1) / kKBlock + 1) : a.nkb;
  // the last key blocks of a causal query block need the element test
  const int nplain = a.causal ? min(nvalid, (kQBlock * i + 1) / kKBlock) : nvalid;
  const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.N;
  const uint8_t* k4 = a.L.k4 + krow0 * ROWB;
  const uint8_t* ke = a.L.ke + krow0 * ROWE;

  // DMA of key block jb into a stage: wave w brings code piece w % NPIECE
  // (the waves past NPIECE bring a copy of the same bytes) and every wave
  // the block's scales, so every wave issues two DMA instructions per block.
  // The scales go as dwords (an LDS DMA of fewer bytes per lane still fills
  // a dword per lane): 64 ROWE / 4 lanes cover them, the others repeat.
  const int piece = wave % NPIECE;
  const int dma_row = piece * (1024 / ROWB) + lane / SLOTS;
  const uint32_t dma_off = dma_row * ROWB + (((lane % SLOTS) ^ swz(dma_row)) * 16);
  const uint32_t dma_eoff = (lane % (kKBlock * ROWE / 4)) * 4;
  auto dma_block = [&](int jb, auto st_c) {
    lds_dma<16>(k4 + (size_t)kKBlock * jb * ROWB + dma_off, stage(st_c) + piece * 1024);
    lds_dma<4>(ke + (size_t)kKBlock * jb * ROWE + dma_eoff, stage(st_c) + CODEB);
  };
  // output stores: a raw buffer over the row's scores; lanes aimed past its
  // end store nothing, so a store needs no branch (a branch would let the
  // compiler move the products around it)
  constexpr uint32_t kNoStore = 0x7fffffffu;

  const int rounds = (a.group + 3) / 4;
  for (int round = 0; round < rounds; ++round) {
    const int g = round * 4 + wave;
    const bool active = g < a.group;  // wave-uniform
    const int hq = hk * a.group + min(g, a.group - 1);
    const size_t bhq = (size_t)b * a.Hq + hq;
    float* out = a.L.scores + (bhq * a.nqb + i) * a.nkb;
    const __amdgpu_buffer_rsrc_t rout = byte_rsrc(out, (uint32_t)a.nkb * 4u);
    // B operand: query row 128 i + 32 rb + l32, channels 64 ks + 32 h + [0, 32);
    // qs[rb] holds the row's scale bytes shifted down by h bytes
    v8i qf[RB][KS];
    int qs[RB];
    if (active) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const size_t qr = bhq * a.N + kQBlock * i + 32 * rb + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 w = *reinterpret_cast<const uint4*>(a.L.q4 + qr * ROWB + 32 * ks + 16 * h);
          qf[rb][ks] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        }
        uint32_t e;
        if constexpr (ROWE == 4) e = *reinterpret_cast<const uint32_t*>(a.L.qe + qr * ROWE);
        else e = *reinterpret_cast<const uint16_t*>(a.L.qe + qr * ROWE);
        qs[rb] = (int)(e >> (8 * h));
      }
    }
    // A 32-key half kb of key block j as A-operand fragments (key
    // 64 j + 32 kb + l32, channels 64 ks + 32 h + [0, 32)) and their E8M0
    // scales (byte 2 ks + h of the key's scales).
    struct KHalf {
      v8i f[KS];
      int e[KS];
    };
    // from global memory (the masked blocks)
    auto load_half = [&](int j, int kb, KHalf& kh) {
      const int row = kKBlock * j + 32 * kb + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = *reinterpret_cast<const uint4*>(k4 + (size_t)row * ROWB + 32 * ks + 16 * h);
        kh.f[ks] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        kh.e[ks] = ke[(size_t)row * ROWE + 2 * ks + h];
      }
    };
    // The same from LDS stage ST (the unmasked blocks); row 32 kb + l32 has
    // the swizzle of row l32. The stage and the half go into the
    // instructions' offset fields; the lane offsets pass an empty asm
    // statement once per pass of the block loop, so that the compiler does
    // not hold a precomputed address per stage instead.
    int frag_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) frag_off[ks] = l32 * ROWB + (((2 * ks + h) ^ swz(l32)) * 16);
    int scale_off = l32 * ROWE + h;
    auto read_half = [&](auto st_c, auto kb_c, KHalf& kh) {
      constexpr int kb = decltype(kb_c)::value;
      const uint8_t* base = stage(st_c);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = *reinterpret_cast<const uint4*>(base + 32 * kb * ROWB + frag_off[ks]);
        kh.f[ks] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        kh.e[ks] = base[CODEB + 32 * kb * ROWE + 2 * ks + scale_off];
      }
    };
    // Per masked (diagonal) key block, this lane's largest estimate with
    // the element test; one half and one row pair at a time (an empty asm
    // statement per group keeps the compiler from issuing all products
    // first), four running maxima keep the chains short.
    auto score_masked = [&](int j) {
      float best[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        KHalf kh;
        load_half(j, kb, kh);
#pragma unroll
        for (int rp = 0; rp < RB; rp += 2) {
          v16f s[2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[u][r] = 0.0f;
          auto step = [&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
#pragma unroll
            for (int u = 0; u < 2; ++u)
              s[u] = mfma_fp4<2 * ks>(kh.f[ks], qf[rp + u][ks], s[u], kh.e[ks], qs[rp + u]);
          };
          step(std::integral_constant<int, 0>{});
          if constexpr (KS == 2) step(std::integral_constant<int, 1>{});
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            // element r: key 64 j + 32 kb + 8 (r/4) + 4 h + r%4, query 128 i + 32 (rp+u) + l32
            const int lim = (32 * (rp + u) + l32) + kQBlock * i - (kKBlock * j + 32 * kb + 4 * h);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 8 * (r >> 2) + (r & 3);
              best[r & 3] = __builtin_fmaxf(best[r & 3], off > lim ? -__builtin_inff() : s[u][r]);
            }
          }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            asm volatile("" : "+v"(best[0]), "+v"(best[1]), "+v"(best[2]), "+v"(best[3]),
                         "+v"(kh.f[ks]));
        }
      }
      return __builtin_fmaxf(__builtin_fmaxf(best[0], best[1]), __builtin_fmaxf(best[2], best[3]));
    };
    auto store_best = [&](int j, float lane_best) {
      const int k = wave_max_key_to_lane63(order_key(lane_best));
      if (lane == 63) out[j] = __int_as_float(order_key(__int_as_float(k)));
    };

    // Unmasked blocks, software-pipelined, through the LDS ring. A block's
    // products go in four groups (group g: 32-key half g / 2, row pair
    // 2 (g % 2)); each product is issued next to a share of the maxima of
    // the group before it (the last group's beside the next block's first),
    // so no vector instruction waits for a matrix result and every matrix
    // instruction has independent vector work beside it. A block's wave
    // reduction runs in steps beside the next block's second and third
    // groups. Each half's fragments are read from the ring one group ahead
    // of their first product. The ring: block j + 3 goes in flight at the
    // barrier of block j (between its second and third groups), which waits
    // for block j + 1; every wave of the workgroup, with a query head or
    // not, keeps this schedule.
    if (nplain > 0) {
      const v16f zero = {};
      constexpr int NM = 2 * KS;   // products per group
      constexpr int NE = 32 / NM;  // estimates per lane taken beside each product
      // product m of group g: u = m % 2 picks the row block of the pair, ks = m / 2
      auto product = [&](const KHalf& kh, auto g_c, auto m_c, v16f (&acc)[2]) {
        constexpr int g = decltype(g_c)::value, m = decltype(m_c)::value;
        constexpr int rp = 2 * (g & 1), u = m & 1, ks = m >> 1;
        if constexpr (ks == 0)
          acc[u] = mfma_fp4<0>(kh.f[0], qf[rp + u][0], zero, kh.e[0], qs[rp + u]);
        else
          acc[u] = mfma_fp4<2>(kh.f[1], qf[rp + u][1], acc[u], kh.e[1], qs[rp + u]);
      };
      // share m of a finished group: its estimates NE m .. NE m + NE - 1 (u = e / 16)
      auto max_share = [&](const v16f (&acc)[2], auto m_c, float (&best)[4]) {
        constexpr int m = decltype(m_c)::value;
#pragma unroll
        for (int e = NE * m; e < NE * m + NE; ++e)
          best[e & 3] = __builtin_fmaxf(best[e & 3], acc[e >> 4][e & 15]);
      };
      auto reset = [](float (&best)[4]) {
#pragma unroll
        for (int x = 0; x < 4; ++x) best[x] = -__builtin_inff();
      };
      auto fold = [](const float (&best)[4]) {
        return __builtin_fmaxf(__builtin_fmaxf(best[0], best[1]), __builtin_fmaxf(best[2], best[3]));
      };
      // step st of block jp's wave reduction (the steps of
      // wave_max_key_to_lane63, then lane 63's store; nothing stored when jp < 0)
      auto red_step = [&](auto st_c, int jp, float (&bprev)[4], int& key) {
        constexpr int st = decltype(st_c)::value;
        if constexpr (st == 0) {
          key = order_key(fold(bprev));
          reset(bprev);
        } else if constexpr (st == 1) key = dpp_max_key<0xB1, 0xF>(key);
        else if constexpr (st == 2) key = dpp_max_key<0x4E, 0xF>(key);
        else if constexpr (st == 3) key = dpp_max_key<0x141, 0xF>(key);
        else if constexpr (st == 4) key = dpp_max_key<0x140, 0xF>(key);
        else if constexpr (st == 5) key = dpp_max_key<0x142, 0xA>(key);
        else if constexpr (st == 6) key = dpp_max_key<0x143, 0xC>(key);
        else {
          const uint32_t voff = (lane == 63 && jp >= 0) ? (uint32_t)jp * 4u : kNoStore;
          __builtin_amdgcn_raw_buffer_store_b32(order_key(__int_as_float(key)), rout, voff, 0, 0);
        }
      };
      // one group's products into acc beside the maxima of prev into best,
      // and reduction steps, half RED of the eight
      auto phase = [&](const KHalf& kh, auto g_c, v16f (&acc)[2], const v16f (&prev)[2],
                       float (&best)[4], auto red_c, int jp, float (&bprev)[4], int& key) {
        constexpr int RED = decltype(red_c)::value;
        static_for<0, NM>([&](auto m_c) {
          constexpr int m = decltype(m_c)::value;
          product(kh, g_c, m_c, acc);
          max_share(prev, m_c, best);
          if constexpr (RED >= 0) {
            constexpr int c = RED * NM + m;
            static_for<8 * c / (2 * NM), 8 * (c + 1) / (2 * NM)>(
                [&](auto st_c) { red_step(st_c, jp, bprev, key); });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      using G0 = std::integral_constant<int, 0>;
      using G1 = std::integral_constant<int, 1>;
      using G2 = std::integral_constant<int, 2>;
      using G3 = std::integral_constant<int, 3>;
      using R0 = std::integral_constant<int, 0>;
      using R1 = std::integral_constant<int, 1>;
      using NoRed = std::integral_constant<int, -1>;
      using KB0 = std::integral_constant<int, 0>;
      using KB1 = std::integral_constant<int, 1>;
      // Vector-memory order: block j issues, after its barrier, block j + 3's
      // two DMA instructions and then (in its third group) the store of
      // block j - 1. At the barrier of block j the operations younger than
      // block j + 1's DMA are therefore the stores of blocks j - 3 and j - 2
      // and block j + 2's DMA: four. The stores of blocks before the first
      // are issued aimed past the end, so the count holds from the start.
      constexpr int kRingWait = waitcnt_imm(4, 0);
      auto sync = [&] {
        __builtin_amdgcn_s_waitcnt(kRingWait);
        __builtin_amdgcn_s_barrier();
      };
      auto dummy_store = [&] { __builtin_amdgcn_raw_buffer_store_b32(0, rout, kNoStore, 0, 0); };
      auto clampj = [&](int j) { return min(j, nplain - 1); };
      dma_block(clampj(0), std::integral_constant<int, 0>{});
      dma_block(clampj(1), std::integral_constant<int, 1>{});
      dummy_store();
      dma_block(clampj(2), std::integral_constant<int, 2>{});
      dummy_store();
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(6, 0));  // block 0
      __builtin_amdgcn_s_barrier();
      if (active) {
        v16f acc0[2], acc1[2];
        float bA[4], bB[4];
        reset(bA);
        reset(bB);
        KHalf h0, h1;
        // Block j (stage ST = j % 4; half 0 in h0 and its first group
        // already in acc0): half 1 of block j into h1, then half 0 of block
        // j + 1 into h0 after the barrier. The first group of block j + 1 is
        // issued even past the last block (clamped blocks are valid memory)
        // and dropped.
        auto block = [&](int j, auto st_c, float (&bcur)[4], float (&bprev)[4]) {
          constexpr int st = decltype(st_c)::value;
          using Next = std::integral_constant<int, (st + 1) % NST>;
          using Ahead = std::integral_constant<int, (st + 3) % NST>;
          int key = 0;
          read_half(st_c, KB1{}, h1);
          phase(h0, G1{}, acc1, acc0, bcur, R0{}, j - 1, bprev, key);
          // the products from h0 are issued before the barrier
          asm volatile("" ::"v"(acc1[0]), "v"(acc1[1]));
          sync();
          dma_block(clampj(j + 3), Ahead{});
          phase(h1, G2{}, acc0, acc1, bcur, R1{}, j - 1, bprev, key);
          read_half(Next{}, KB0{}, h0);
          phase(h1, G3{}, acc1, acc0, bcur, NoRed{}, j, bprev, key);
          phase(h0, G0{}, acc0, acc1, bcur, NoRed{}, j, bprev, key);
          // the next block's first products stay ahead of the loop's exit test
          asm volatile("" ::"v"(acc0[0]), "v"(acc0[1]));
        };
        read_half(std::integral_constant<int, 0>{}, KB0{}, h0);
        static_for<0, NM>([&](auto m_c) { product(h0, G0{}, m_c, acc0); });
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        for (int j = 0;; j += 4) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(frag_off[ks]));
          asm volatile("" : "+v"(scale_off));
          block(j, S0{}, bA, bB);
          if (j + 1 == nplain) {
            store_best(j, fold(bA));
            break;
          }
          block(j + 1, S1{}, bB, bA);
          if (j + 2 == nplain) {
            store_best(j + 1, fold(bB));
            break;
          }
          block(j + 2, S2{}, bA, bB);
          if (j + 3 == nplain) {
            store_best(j + 2, fold(bA));
            break;
          }
          block(j + 3, S3{}, bB, bA);
          if (j + 4 == nplain) {
            store_best(j + 3, fold(bB));
            break;
          }
        }
      } else {
        // no query head: the same barriers, DMA and vector-memory order
        for (int j = 0; j < nplain; j += NST) {
          static_for<0, NST>([&](auto x_c) {
            constexpr int x = decltype(x_c)::value;
            if (j + x < nplain) {
              sync();
              dma_block(clampj(j + x + 3), std::integral_constant<int, (x + 3) % NST>{});
              dummy_store();
            }
          });
        }
      }
      // the ring is free for the next round once every DMA has landed and
      // every wave has read its last block
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      __builtin_amdgcn_s_barrier();
    }
    // the masked blocks, one at a time
    if (active) {
      for (int j = nplain; j < nvalid; ++j) {
        store_best(j, score_masked(j));
      }
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
