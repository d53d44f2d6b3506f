// Microbenchmarks that measure the roofline denominators on the part itself (gfx950):
// the dense block-scaled fp4 MFMA rate, the issue rates of the vector instructions the
// attention kernel's softmax is made of, the core clock under load, and HBM streaming
// bandwidth.  The benchmark reports its kernels against these measured figures beside
// the published peaks.  Nothing here is used by the attention path.
//
// Every probe kernel reads s_memtime (core-clock counter) and s_memrealtime (constant
// wall-clock counter) around its timed loop; each wave adds its two deltas to
// stats[0] and stats[1] and counts itself in stats[2], so the ratio of the sums is the
// core clock in units of the wall-clock rate.  stats (4 x uint64, device memory) must
// be zero on entry.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void record(unsigned long long* st, unsigned long long c0, unsigned long long w0,
                                       float keep) {
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long w1 = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&st[0], c1 - c0);
    atomicAdd(&st[1], w1 - w0);
    atomicAdd(&st[2], 1ull);
    // the results must stay live; this comparison is never true for the values the probes make
    if (keep == 1234.5f) atomicAdd(&st[3], 1ull);
  }
}

// Four independent accumulator chains of 32x32x64 fp4 x fp4 MFMAs (E8M0 scales), issued
// back to back: 4 * iters MFMAs per wave, 2 * 32 * 32 * 64 flop each.
__global__ __launch_bounds__(256) void k_mfma_fp4(int64_t iters, int code, int scale, unsigned long long* st) {
  const v8i a = {code, code, code, code, 0, 0, 0, 0};
  const v8i b = {code ^ (int)threadIdx.x, code, code, code, 0, 0, 0, 0};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, scale, 0, scale);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 4, 4, 0, scale, 0, scale);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 4, 4, 0, scale, 0, scale);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 4, 4, 0, scale, 0, scale);
  }
  float keep = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) keep += c0[v] + c1[v] + c2[v] + c3[v];
  record(st, t0, w0, keep);
}

// Eight independent chains of one vector instruction, 32 instructions per loop trip:
// 32 * iters instructions per wave.  The instruction is written out so that exactly it
// is timed (the compiler may not fold or reorder the chains).
enum { P_EXP = 0, P_CVT_FP4 = 1, P_FMA = 2, P_MAX3 = 3 };

template <int KIND>
__device__ __forceinline__ void op(float& x, uint32_t& r, float y, float a, float b, float s) {
  if constexpr (KIND == P_EXP) asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x));
  if constexpr (KIND == P_CVT_FP4) asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(r) : "v"(x), "v"(y), "v"(s));
  if constexpr (KIND == P_FMA) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
  if constexpr (KIND == P_MAX3) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
}

template <int KIND>
__global__ __launch_bounds__(256) void k_valu(int64_t iters, float seed, unsigned long long* st) {
  float x[8];
  uint32_t r[8];
  const float a = 0.999f + 1e-7f * (float)threadIdx.x, b = 1e-3f * seed, s = 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = seed * (float)(j + 1) + 1e-3f * (float)threadIdx.x;
    r[j] = (uint32_t)j;
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) op<KIND>(x[j], r[j], x[(j + 1) & 7], a, b, s);
  }
  float keep = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) keep += x[j] + (float)r[j];
  record(st, t0, w0, keep);
}

// HBM streaming: 16-byte non-temporal loads, four in flight per thread per trip.
__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ p, int64_t n16, unsigned* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(p + i);
    const u32x4 v1 = __builtin_nontemporal_load(p + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never written
}

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    dst[i] = v0;
    dst[i + stride] = v1;
    dst[i + 2 * stride] = v2;
    dst[i + 3 * stride] = v3;
  }
  for (; i < n16; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

// Compute units of the current device, and the rate (kHz) of the s_memrealtime counter.
int32_t mxprobe_cu_count(void) { return cu_count(); }

int32_t mxprobe_wall_clock_khz(void) {
  int dev = 0, r = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return r;
}

// Returns 0, -1 for bad arguments, -4 for a launch error.  waves_per_simd: 1..8 (one
// 4-wave workgroup per compute unit and wave per SIMD).
int32_t mxprobe_mfma_fp4(int64_t iters, int32_t waves_per_simd, uint64_t* stats, void* stream) {
  const int cus = cu_count();
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8 || !stats || cus < 1) return -1;
  hipLaunchKernelGGL(k_mfma_fp4, dim3(cus * waves_per_simd), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     0x22222222, 127, reinterpret_cast<unsigned long long*>(stats));
  return status(hipGetLastError());
}

// kind: 0 v_exp_f32, 1 v_cvt_scalef32_pk_fp4_f32, 2 v_fma_f32, 3 v_max3_f32.
int32_t mxprobe_valu(int32_t kind, int64_t iters, int32_t waves_per_simd, uint64_t* stats, void* stream) {
  const int cus = cu_count();
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8 || !stats || cus < 1) return -1;
  const dim3 g(cus * waves_per_simd), b(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* st = reinterpret_cast<unsigned long long*>(stats);
  switch (kind) {
    case P_EXP: hipLaunchKernelGGL(k_valu<P_EXP>, g, b, 0, s, iters, 0.5f, st); break;
    case P_CVT_FP4: hipLaunchKernelGGL(k_valu<P_CVT_FP4>, g, b, 0, s, iters, 0.5f, st); break;
    case P_FMA: hipLaunchKernelGGL(k_valu<P_FMA>, g, b, 0, s, iters, 0.5f, st); break;
    case P_MAX3: hipLaunchKernelGGL(k_valu<P_MAX3>, g, b, 0, s, iters, 0.5f, st); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

// bytes: a multiple of 16; src (and dst) 16-byte aligned device memory of that size.
int32_t mxprobe_hbm_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  const int cus = cu_count();
  if (!src || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || cus < 1) return -1;
  hipLaunchKernelGGL(k_read, dim3(cus * 8), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return status(hipGetLastError());
}

int32_t mxprobe_hbm_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  const int cus = cu_count();
  if (!src || !dst || bytes == 0 || bytes % 16 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) ||
      cus < 1)
    return -1;
  hipLaunchKernelGGL(k_copy, dim3(cus * 8), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (int64_t)(bytes / 16));
  return status(hipGetLastError());
}

}  // extern "C"
