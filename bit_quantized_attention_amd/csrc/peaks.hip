// Micro-benchmarks of the MI355X (gfx950) rates that bound the attention
// kernel: INT8 and BF16 matrix instructions and their 1:2 mix (the attention's
// ratio), fp32 FMA and exp2 on the vector unit, matrix / vector co-issue from
// one wave, LDS reads (16-byte and 8-byte transposing), and an HBM copy.
//
// Built into its own library (libqattn_peaks.so), used only by the benchmark:
//   int qattn_peak(int kind, int param, double* result)
// result[0] = rate (operations, lane-instructions or bytes per second, see
// kind), result[1] = mean kernel time in ms, result[2] = shader clock in GHz
// (s_memtime ticks over s_memrealtime ticks of the first wave, under load),
// result[3] = cycles per loop iteration of that wave (s_memtime).
// Returns 0, or a HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

enum Kind {
  kMfmaI8 = 0,      // v_mfma_i32_32x32x32_i8, 8 independent accumulators
  kMfmaBf16 = 1,    // v_mfma_f32_32x32x16_bf16, 8 independent accumulators
  kMfmaMix = 2,     // per iteration 2 INT8 + 4 BF16 (the attention's 1:2)
  kValuFma = 3,     // v_fma_f32, 8 chains per lane
  kValuExp = 4,     // v_exp_f32, 8 chains per lane
  kCoissueExp = 5,  // per BF16 matrix instruction, `param` independent v_exp_f32 (1 wave per SIMD)
  kCoissueFma = 6,  // per BF16 matrix instruction, `param` independent v_fma_f32 (1 wave per SIMD)
  kLdsB128 = 7,     // ds_read_b128
  kLdsTr16 = 8,     // ds_read_b64_tr_b16
  kCopy = 9,        // 1 GiB device copy, 16 bytes per lane
  kCoissue16 = 10,  // per v_mfma_f32_16x16x32_bf16, `param` independent v_fma_f32 (1 wave per SIMD)
  kCoissueI8 = 11,  // per v_mfma_i32_32x32x32_i8, `param` independent v_fma_f32 (1 wave per SIMD)
  kSplitFma = 12,   // two waves per SIMD: one issues BF16 matrix instructions only, the
                    // other `param` v_fma_f32 per matrix instruction of its partner
  kSplitExp = 13,   // the same with v_exp_f32
  kMfmaFp4 = 14,    // v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands, 8 accumulators
  kMfmaFp4Vs = 15,  // the same with per-lane E8M0 scales in VGPRs
};

struct Clock {
  uint64_t t0, r0;
};

__device__ __forceinline__ Clock clock_start() {
  Clock c;
  c.t0 = __builtin_amdgcn_s_memtime();
  c.r0 = __builtin_amdgcn_s_memrealtime();
  return c;
}

__device__ __forceinline__ void clock_stop(const Clock& c, unsigned long long* out) {
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = t1 - c.t0;
    out[1] = r1 - c.r0;
  }
}

template <typename T>
__device__ __forceinline__ void keep(T& v) {
  asm volatile("" : "+v"(v));
}

__global__ __launch_bounds__(256) void k_mfma_i8(int iters, unsigned long long* clk, int* sink) {
  v4i a = {(int)threadIdx.x, 3, 5, 7}, b = {11, (int)threadIdx.x, 13, 17};
  v16i c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = j + r;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  }
  clock_stop(ck, clk);
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= c[j][r];
  if (s == 0x7fffffff) sink[0] = s;
}

__global__ __launch_bounds__(256) void k_mfma_bf16(int iters, unsigned long long* clk, int* sink) {
  v8bf a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)(threadIdx.x + e);
    b[e] = (__bf16)(float)(e - (int)threadIdx.x);
  }
  v16f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = (float)(j + r);
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 1.2345f) sink[0] = 1;
}

__global__ __launch_bounds__(256) void k_mfma_mix(int iters, unsigned long long* clk, int* sink) {
  v4i a = {(int)threadIdx.x, 3, 5, 7}, b = {11, (int)threadIdx.x, 13, 17};
  v8bf x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (__bf16)(float)(threadIdx.x + e);
    y[e] = (__bf16)(float)(e - (int)threadIdx.x);
  }
  v16i ci[2];
  v16f cf[4];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ci[0][r] = r;
    ci[1][r] = 2 * r;
#pragma unroll
    for (int j = 0; j < 4; ++j) cf[j][r] = (float)(j * r);
  }
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
    ci[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, ci[0], 0, 0, 0);
    cf[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, cf[0], 0, 0, 0);
    cf[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, cf[1], 0, 0, 0);
    ci[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, ci[1], 0, 0, 0);
    cf[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, cf[2], 0, 0, 0);
    cf[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, cf[3], 0, 0, 0);
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s += (float)(ci[0][r] ^ ci[1][r]);
#pragma unroll
    for (int j = 0; j < 4; ++j) s += cf[j][r];
  }
  if (s == 1.2345f) sink[0] = 1;
}

__global__ __launch_bounds__(256) void k_valu_fma(int iters, unsigned long long* clk, int* sink) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)(threadIdx.x * 8 + j) * 1e-3f;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 0.25f);
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  if (s == 1.2345f) sink[0] = 1;
}

__global__ __launch_bounds__(256) void k_valu_exp(int iters, unsigned long long* clk, int* sink) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -(float)(threadIdx.x * 8 + j) * 1e-3f;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = __builtin_amdgcn_exp2f(x[j]);
      keep(x[j]);
    }
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  if (s == 1.2345f) sink[0] = 1;
}

// One wave per SIMD (launch bounds 256, one workgroup per CU through its LDS
// size): per iteration 4 BF16 matrix instructions on independent accumulators,
// each followed by NV independent vector instructions (exp2 or fma).
template <int NV, bool EXP>
__global__ __launch_bounds__(256) void k_coissue(int iters, unsigned long long* clk, int* sink) {
  extern __shared__ int lds_pad[];
  v8bf a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)(threadIdx.x + e);
    b[e] = (__bf16)(float)(e - (int)threadIdx.x);
  }
  v16f c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = (float)(j + r);
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = -(float)(threadIdx.x * 16 + j) * 1e-4f;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        float& v = x[(j * NV + e) & 15];
        if constexpr (EXP) v = __builtin_amdgcn_exp2f(v);
        else v = __builtin_fmaf(v, 0.999f, 0.25f);
        keep(v);
      }
      // keep each matrix instruction with its own vector instructions
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  if (s == 1.2345f) sink[0] = (int)lds_pad[threadIdx.x];
}

template <bool VSCALE>
__global__ __launch_bounds__(256) void k_mfma_fp4(int iters, unsigned long long* clk, int* sink) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i a = {(int)threadIdx.x, 0x11111111, 0x22222222, 0x01234567, 0, 0, 0, 0};
  const v8i b = {0x76543210, (int)threadIdx.x, 0x13572468, 0x24681357, 0, 0, 0, 0};
  v16f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = (float)(j + r);
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
    {
      if constexpr (VSCALE) {
        int sa = 126 + (int)(threadIdx.x & 1), sb = 127 - (int)((threadIdx.x >> 1) & 1);
        keep(sa);
        keep(sb);
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 4, 4, 0, sa, 0, sb);
      } else {
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 4, 4, 0, 127, 0, 127);
      }
    }
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 1.2345f) sink[0] = 1;
}

// One wave per SIMD: per iteration 8 16x16x32 BF16 matrix instructions (16
// cycles each) on independent accumulators, each followed by NV vector fmas.
template <int NV>
__global__ __launch_bounds__(256) void k_coissue16(int iters, unsigned long long* clk, int* sink) {
  extern __shared__ int lds_pad[];
  v8bf a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)(threadIdx.x + e);
    b[e] = (__bf16)(float)(e - (int)threadIdx.x);
  }
  v4f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) c[j][r] = (float)(j + r);
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = -(float)(threadIdx.x * 16 + j) * 1e-4f;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        float& v = x[(j * NV + e) & 15];
        v = __builtin_fmaf(v, 0.999f, 0.25f);
        keep(v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  clock_stop(ck, clk);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += c[j][r];
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  if (s == 1.2345f) sink[0] = (int)lds_pad[threadIdx.x];
}

// One wave per SIMD: per iteration 4 INT8 32x32x32 matrix instructions, each
// followed by NV vector fmas.
template <int NV>
__global__ __launch_bounds__(256) void k_coissue_i8(int iters, unsigned long long* clk, int* sink) {
  extern __shared__ int lds_pad[];
  v4i a = {(int)threadIdx.x, 3, 5, 7}, b = {11, (int)threadIdx.x, 13, 17};
  v16i c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = j + r;
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = -(float)(threadIdx.x * 16 + j) * 1e-4f;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        float& v = x[(j * NV + e) & 15];
        v = __builtin_fmaf(v, 0.999f, 0.25f);
        keep(v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  clock_stop(ck, clk);
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= c[j][r];
  float f = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) f += x[j];
  if (s == 0x7fffffff || f == 1.2345f) sink[0] = (int)lds_pad[threadIdx.x];
}

// Two waves per SIMD (8 waves, one workgroup per CU): waves 0-3 issue only
// BF16 32x32x16 matrix instructions (4 per iteration), waves 4-7 only vector
// instructions (4 * NV per iteration: fma or exp2). The first wave's clock
// gives the matrix waves' time per iteration.
template <int NV, bool EXP>
__global__ __launch_bounds__(512) void k_split(int iters, unsigned long long* clk, int* sink) {
  extern __shared__ int lds_pad[];
  const int wave = threadIdx.x >> 6;
  const Clock ck = clock_start();
  if (wave < 4) {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)(threadIdx.x + e);
      b[e] = (__bf16)(float)(e - (int)threadIdx.x);
    }
    v16f c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[j][r] = (float)(j + r);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    clock_stop(ck, clk);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += c[j][r];
    if (s == 1.2345f) sink[0] = (int)lds_pad[threadIdx.x];
  } else {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = -(float)(threadIdx.x * 16 + j) * 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int e = 0; e < 4 * NV; ++e) {
        float& v = x[e & 15];
        if constexpr (EXP) v = __builtin_amdgcn_exp2f(v);
        else v = __builtin_fmaf(v, 0.999f, 0.25f);
        keep(v);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
    if (s == 1.2345f) sink[0] = 2;
  }
}

// LDS reads: 8 reads in flight per lane per iteration over a 64 KiB buffer;
// consecutive lanes read consecutive 16-byte (8-byte) slots.
template <bool TR>
__global__ __launch_bounds__(256) void k_lds(int iters, unsigned long long* clk, int* sink) {
  __shared__ __attribute__((aligned(16))) int8_t buf[65536];
  for (int i = threadIdx.x; i < 65536 / 4; i += 256) reinterpret_cast<int*>(buf)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int acc = 0;
  const Clock ck = clock_start();
  for (int i = 0; i < iters; ++i) {
    if constexpr (TR) {
      v4s r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int off = (((i * 8 + j) * 4 + wave) * 512 + lane * 8) & 0xFFFF;
        keep(off);  // opaque: every read is issued
        r[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(buf + off));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= r[j][0] ^ r[j][3];
    } else {
      v4i r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int off = (((i * 8 + j) * 4 + wave) * 1024 + lane * 16) & 0xFFFF;
        keep(off);  // opaque: every read is issued
        r[j] = *reinterpret_cast<const v4i*>(buf + off);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= r[j][0] ^ r[j][3];
    }
  }
  clock_stop(ck, clk);
  if (acc == 0x7fffffff) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int qattn_peak(int kind, int param, double* result) {
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  const int ncu = prop.multiProcessorCount;
  unsigned long long* clk = nullptr;
  int* sink = nullptr;
  hipError_t e = hipMalloc(&clk, 2 * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMalloc(&sink, sizeof(int));
  if (e != hipSuccess) return (int)e;
  void* src = nullptr;
  void* dst = nullptr;
  const size_t copy_bytes = (size_t)1 << 30;
  if (kind == kCopy) {
    e = hipMalloc(&src, copy_bytes);
    if (e == hipSuccess) e = hipMalloc(&dst, copy_bytes);
    if (e == hipSuccess) e = hipMemset(src, 1, copy_bytes);
    if (e != hipSuccess) return (int)e;
  }
  // two workgroups of 4 waves per CU (two waves per SIMD), many rounds
  const int blocks = 2 * ncu;
  int iters = 0;
  double per_iter = 0.0;  // operations / lane-instructions / bytes per iteration per workgroup
  auto launch = [&]() -> hipError_t {
    switch (kind) {
      case kMfmaI8:
        iters = 20000;
        per_iter = 4.0 * 8 * 65536.0;
        hipLaunchKernelGGL(k_mfma_i8, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kMfmaBf16:
        iters = 20000;
        per_iter = 4.0 * 8 * 32768.0;
        hipLaunchKernelGGL(k_mfma_bf16, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kMfmaMix:
        iters = 20000;
        per_iter = 4.0 * (2 * 65536.0 + 4 * 32768.0);
        hipLaunchKernelGGL(k_mfma_mix, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kValuFma:
        iters = 100000;
        per_iter = 256.0 * 8;
        hipLaunchKernelGGL(k_valu_fma, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kValuExp:
        iters = 50000;
        per_iter = 256.0 * 8;
        hipLaunchKernelGGL(k_valu_exp, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kCoissueExp:
      case kCoissueFma: {
        iters = 20000;
        per_iter = 4.0 * 4 * 32768.0;  // matrix flops; the vector work rides along
        const size_t lds = 96 * 1024;  // one workgroup per CU: one wave per SIMD
        const bool ex = kind == kCoissueExp;
#define QP_CO(NV)                                                                                    \
  case NV:                                                                                         \
    if (ex) hipLaunchKernelGGL((k_coissue<NV, true>), dim3(ncu), dim3(256), lds, 0, iters, clk, sink); \
    else hipLaunchKernelGGL((k_coissue<NV, false>), dim3(ncu), dim3(256), lds, 0, iters, clk, sink);  \
    break;
        switch (param) {
          QP_CO(0)
          QP_CO(2)
          QP_CO(4)
          QP_CO(6)
          QP_CO(8)
          QP_CO(12)
          QP_CO(16)
          default:
            return hipErrorInvalidValue;
        }
#undef QP_CO
        break;
      }
      case kCoissue16:
      case kCoissueI8: {
        iters = 20000;
        const size_t lds = 96 * 1024;
        const bool i8 = kind == kCoissueI8;
        per_iter = i8 ? 4.0 * 4 * 65536.0 : 4.0 * 8 * 16384.0;
#define QP_C2(NV)                                                                                      \
  case NV:                                                                                           \
    if (i8) hipLaunchKernelGGL((k_coissue_i8<NV>), dim3(ncu), dim3(256), lds, 0, iters, clk, sink);  \
    else hipLaunchKernelGGL((k_coissue16<NV>), dim3(ncu), dim3(256), lds, 0, iters, clk, sink);      \
    break;
        switch (param) {
          QP_C2(0)
          QP_C2(1)
          QP_C2(2)
          QP_C2(3)
          QP_C2(4)
          QP_C2(6)
          QP_C2(8)
          default:
            return hipErrorInvalidValue;
        }
#undef QP_C2
        break;
      }
      case kSplitFma:
      case kSplitExp: {
        iters = 20000;
        per_iter = 4.0 * 4 * 32768.0;  // the matrix waves' flops
        const size_t lds = 96 * 1024;
        const bool ex = kind == kSplitExp;
#define QP_SP(NV)                                                                                        \
  case NV:                                                                                             \
    if (ex) hipLaunchKernelGGL((k_split<NV, true>), dim3(ncu), dim3(512), lds, 0, iters, clk, sink);     \
    else hipLaunchKernelGGL((k_split<NV, false>), dim3(ncu), dim3(512), lds, 0, iters, clk, sink);       \
    break;
        switch (param) {
          QP_SP(0)
          QP_SP(2)
          QP_SP(4)
          QP_SP(6)
          QP_SP(8)
          default:
            return hipErrorInvalidValue;
        }
#undef QP_SP
        break;
      }
      case kMfmaFp4:
        iters = 20000;
        per_iter = 4.0 * 8 * 131072.0;
        hipLaunchKernelGGL(k_mfma_fp4<false>, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kMfmaFp4Vs:
        iters = 20000;
        per_iter = 4.0 * 8 * 131072.0;
        hipLaunchKernelGGL(k_mfma_fp4<true>, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kLdsB128:
        iters = 20000;
        per_iter = 256.0 * 8 * 16;
        hipLaunchKernelGGL(k_lds<false>, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kLdsTr16:
        iters = 20000;
        per_iter = 256.0 * 8 * 8;
        hipLaunchKernelGGL(k_lds<true>, dim3(blocks), dim3(256), 0, 0, iters, clk, sink);
        break;
      case kCopy:
        iters = 1;
        per_iter = 0.0;
        hipLaunchKernelGGL(k_copy, dim3(8 * ncu), dim3(256), 0, 0, (const uint4*)src, (uint4*)dst,
                           copy_bytes / 16);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  };
  // warm-up, then 5 timed launches
  e = launch();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  hipEvent_t a, b;
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  const int reps = 5;
  if (e == hipSuccess) e = hipEventRecord(a, 0);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, 0);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  unsigned long long ck[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpy(ck, clk, sizeof(ck), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    const double t = ms / reps;
    const bool one_per_cu = kind == kCoissueExp || kind == kCoissueFma || kind == kCoissue16 ||
                            kind == kCoissueI8 || kind == kSplitFma || kind == kSplitExp;
    const int nblk = one_per_cu ? ncu : blocks;
    const double work = kind == kCopy ? 2.0 * copy_bytes : per_iter * iters * nblk;
    result[0] = work / (t * 1e-3);
    result[1] = t;
    result[2] = ck[1] ? (double)ck[0] / (double)ck[1] * 0.1 : 0.0;
    result[3] = iters ? (double)ck[0] / iters : 0.0;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  (void)hipFree(clk);
  (void)hipFree(sink);
  if (src) (void)hipFree(src);
  if (dst) (void)hipFree(dst);
  return (int)e;
}
