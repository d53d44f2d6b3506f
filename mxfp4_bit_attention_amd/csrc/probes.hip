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

// MFMA operands: with RAND, four sets of pseudo-random fp4 codes per lane (a counter hash),
// one per accumulator chain, so that successive MFMAs see different bits as they do on real
// data (the part's clock under load depends on how much the operands toggle); otherwise one
// constant pattern.
struct Operands {
  v8i a[4], b[4];
};
template <bool RAND>
__device__ __forceinline__ Operands operands(int code) {
  Operands o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t h = (threadIdx.x + 256u * blockIdx.x) * 0x9E3779B9u + (uint32_t)k * 0x85EBCA6Bu;
    int w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h ^= h >> 15;
      h *= 0x2C1B3C6Du;
      h ^= h >> 12;
      w[e] = RAND ? (int)h : code;
    }
    o.a[k] = v8i{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
    o.b[k] = v8i{RAND ? w[4] : code ^ (int)threadIdx.x, w[5], w[6], w[7], 0, 0, 0, 0};
  }
  return o;
}

// Four independent accumulator chains of 32x32x64 fp4 x fp4 MFMAs (E8M0 scales), issued
// back to back: 4 * iters MFMAs per wave, 2 * 32 * 32 * 64 flop each.
template <bool RAND>
__global__ __launch_bounds__(256) void k_mfma_fp4(int64_t iters, int code, int scale, unsigned long long* st) {
  const Operands o = operands<RAND>(code);
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[0], o.b[0], c0, 4, 4, 0, scale, 0, scale);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[1], o.b[1], c1, 4, 4, 0, scale, 0, scale);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[2], o.b[2], c2, 4, 4, 0, scale, 0, scale);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[3], o.b[3], c3, 4, 4, 0, scale, 0, scale);
  }
  float keep = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) keep += c0[v] + c1[v] + c2[v] + c3[v];
  record(st, t0, w0, keep);
}

// Eight independent chains of one vector instruction, 32 instructions per loop trip:
// 32 * iters instructions per wave.  The instruction is written out so that exactly it
// is timed (the compiler may not fold or reorder the chains).
// P_EXP_FMA alternates the two (16 of each per trip): its time against the sum of the
// two alone shows whether exponentials and FMAs overlap on a SIMD.
enum { P_EXP = 0, P_CVT_FP4 = 1, P_FMA = 2, P_MAX3 = 3, P_EXP_FMA = 4 };

template <int KIND>
__device__ __forceinline__ void op(float& x, uint32_t& r, float y, float a, float b, float s, int j) {
  if constexpr (KIND == P_EXP) asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x));
  if constexpr (KIND == P_CVT_FP4) asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(r) : "v"(x), "v"(y), "v"(s));
  if constexpr (KIND == P_FMA) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
  if constexpr (KIND == P_MAX3) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
  if constexpr (KIND == P_EXP_FMA) {
    if (j & 1) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b));
    else asm volatile("v_exp_f32_e64 %0, -%0" : "+v"(x));
  }
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
      for (int j = 0; j < 8; ++j) op<KIND>(x[j], r[j], x[(j + 1) & 7], a, b, s, j);
  }
  float keep = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) keep += x[j] + (float)r[j];
  record(st, t0, w0, keep);
}

// The attention kernel's per-tile instruction mix with no memory, LDS or barrier: per
// trip and wave, NMFMA fp4 32x32x64 MFMAs (four accumulator chains; 18 at d = 128, 10 at
// d = 64), 65 v_exp_f32, 32 fp4 conversions, 65 fp32 FMAs and 34 NaN-propagating max3,
// the counts of one 32-query x 128-key tile of the attention's inner loop.  With three
// waves per SIMD, as the attention kernel runs, its time per trip is the cost of that mix
// on its own.  VALU = false keeps only the MFMAs, NMFMA = 0 only the vector instructions:
// the two parts alone against the whole show how much of the MFMA time the vector work
// hides.
template <int NMFMA, bool VALU = true, bool RAND = false>
__global__ __launch_bounds__(256, 3) void k_mix(int64_t iters, int code, unsigned long long* st) {
  const Operands o = operands<RAND>(code);
  v16f c[4] = {};
  float x[8], y[8], z[8];
  uint32_t r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = 0.25f * (float)(j + 1) + 1e-3f * (float)threadIdx.x;
    y[j] = 0.5f + 1e-3f * (float)(j + threadIdx.x);
    z[j] = -1.0f;
    r[j] = (uint32_t)j;
  }
  const float fa = 0.999f, fb = 1e-3f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < NMFMA; ++k)
      c[k & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[k & 3], o.b[k & 3], c[k & 3], 4, 4, 0, 127, 0, 127);
    if constexpr (VALU) {
      // the max3 operands change every step, so no two of them can be folded
#pragma unroll
      for (int k = 0; k < 65; ++k) {
        x[k & 7] = __builtin_amdgcn_exp2f(-x[k & 7]);
        y[k & 7] = __builtin_fmaf(y[k & 7], fa, fb);
        if (k < 34)
          z[k & 7] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(z[k & 7], x[k & 7]), y[k & 7]);
      }
#pragma unroll
      for (int k = 0; k < 32; k += 4) {
        r[k & 7] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r[k & 7], x[k & 7], y[k & 7], 1.0f, 0);
        r[k & 7] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r[k & 7], x[(k + 1) & 7], y[(k + 1) & 7], 1.0f, 1);
        r[(k + 1) & 7] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r[(k + 1) & 7], x[(k + 2) & 7], y[(k + 2) & 7], 1.0f, 2);
        r[(k + 1) & 7] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r[(k + 1) & 7], x[(k + 3) & 7], y[(k + 3) & 7], 1.0f, 3);
      }
    }
  }
  float keep = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) keep += x[j] + y[j] + z[j] + (float)r[j];
#pragma unroll
  for (int v = 0; v < 16; ++v) keep += c[0][v] + c[1][v] + c[2][v] + c[3][v];
  record(st, t0, w0, keep);
}

// HBM streaming through global->LDS DMA (buffer_load ... lds with the non-temporal policy,
// the path the quantisers read their input by): each wave moves 8 KB per trip into its own
// LDS slot.  COPY also reads the slot back and stores it to dst with ordinary stores.
typedef __attribute__((address_space(3))) void lds_void;

template <bool COPY>
__global__ __launch_bounds__(256) void k_stream_dma(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int64_t chunks, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[4 * 8192];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* mine = buf + 8192 * wave;
  const int64_t nw = (int64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (int64_t ch = (int64_t)blockIdx.x * 4 + wave; ch < chunks; ch += nw) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + ch * 8192), (short)0, 8192, 0x00020000);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(mine + 1024 * u), 16, (uint32_t)(1024 * u + 16 * lane),
                                               0, 0, 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMAs have landed
    if constexpr (COPY) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(mine + 1024 * u + 16 * lane);
        *reinterpret_cast<u32x4*>(dst + ch * 8192 + 1024 * u + 16 * lane) = v;
      }
    } else {
      acc ^= *reinterpret_cast<const uint32_t*>(mine + 4 * lane);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (!COPY && acc == 0x9E3779B9u) sink[0] = acc;  // keeps the reads; practically never written
}

// HBM streaming: 16-byte non-temporal loads, eight in flight per thread per trip.
__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ p, int64_t n16, unsigned* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never written
}

template <bool NT_STORE>
__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (NT_STORE) __builtin_nontemporal_store(v[u], dst + i + u * stride);
      else dst[i + u * stride] = v[u];
    }
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
int32_t mxprobe_mfma_fp4(int64_t iters, int32_t waves_per_simd, int32_t random_operands, uint64_t* stats,
                         void* stream) {
  const int cus = cu_count();
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8 || !stats || cus < 1) return -1;
  const dim3 g(cus * waves_per_simd), b(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* st = reinterpret_cast<unsigned long long*>(stats);
  if (random_operands) hipLaunchKernelGGL(k_mfma_fp4<true>, g, b, 0, s, iters, 0x22222222, 127, st);
  else hipLaunchKernelGGL(k_mfma_fp4<false>, g, b, 0, s, iters, 0x22222222, 127, st);
  return status(hipGetLastError());
}

// kind: 0 v_exp_f32, 1 v_cvt_scalef32_pk_fp4_f32, 2 v_fma_f32, 3 v_max3_f32, 4 v_exp_f32 and
// v_fma_f32 alternating.
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
    case P_EXP_FMA: hipLaunchKernelGGL(k_valu<P_EXP_FMA>, g, b, 0, s, iters, 0.5f, st); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

// The attention tile's instruction mix (k_mix) for head dimension d (128 or 64), three
// waves per SIMD.  part: 0 the whole mix, 1 its vector instructions only, 2 its MFMAs only,
// 3 the whole mix with pseudo-random MFMA operands (d = 128 only).
int32_t mxprobe_mix(int64_t iters, int32_t d, int32_t part, uint64_t* stats, void* stream) {
  const int cus = cu_count();
  if (iters < 1 || !stats || cus < 1 || (d != 128 && d != 64) || part < 0 || part > 3 || (part == 3 && d != 128))
    return -1;
  unsigned long long* st = reinterpret_cast<unsigned long long*>(stats);
  const dim3 g(cus * 3), b(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (part == 3) hipLaunchKernelGGL((k_mix<18, true, true>), g, b, 0, s, iters, 0x22222222, st);
  else if (part == 1) hipLaunchKernelGGL((k_mix<0, true>), g, b, 0, s, iters, 0x22222222, st);
  else if (d == 128 && part == 0) hipLaunchKernelGGL((k_mix<18, true>), g, b, 0, s, iters, 0x22222222, st);
  else if (d == 128) hipLaunchKernelGGL((k_mix<18, false>), g, b, 0, s, iters, 0x22222222, st);
  else if (part == 0) hipLaunchKernelGGL((k_mix<10, true>), g, b, 0, s, iters, 0x22222222, st);
  else hipLaunchKernelGGL((k_mix<10, false>), g, b, 0, s, iters, 0x22222222, st);
  return status(hipGetLastError());
}

// Global->LDS DMA stream: bytes a multiple of 8192; copy = 0 reads only.
int32_t mxprobe_hbm_dma(const void* src, void* dst, uint64_t bytes, int32_t blocks_per_cu, int32_t copy,
                        uint32_t* sink, void* stream) {
  const int cus = cu_count();
  if (!src || !sink || (copy && !dst) || bytes == 0 || bytes % 8192 || cus < 1 || blocks_per_cu < 1 ||
      blocks_per_cu > 64)
    return -1;
  const dim3 g(cus * blocks_per_cu), b(256);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  if (copy) hipLaunchKernelGGL(k_stream_dma<true>, g, b, 0, static_cast<hipStream_t>(stream), s, d, (int64_t)(bytes / 8192), sink);
  else hipLaunchKernelGGL(k_stream_dma<false>, g, b, 0, static_cast<hipStream_t>(stream), s, d, (int64_t)(bytes / 8192), sink);
  return status(hipGetLastError());
}

// bytes: a multiple of 16; src (and dst) 16-byte aligned device memory of that size.
// blocks_per_cu: 1..64 workgroups of 256 threads per compute unit.  nt_store: store
// with the non-temporal cache policy.
int32_t mxprobe_hbm_read(const void* src, uint64_t bytes, int32_t blocks_per_cu, uint32_t* sink, void* stream) {
  const int cus = cu_count();
  if (!src || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || cus < 1 ||
      blocks_per_cu < 1 || blocks_per_cu > 64)
    return -1;
  hipLaunchKernelGGL(k_read, dim3(cus * blocks_per_cu), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return status(hipGetLastError());
}

int32_t mxprobe_hbm_copy(const void* src, void* dst, uint64_t bytes, int32_t blocks_per_cu, int32_t nt_store,
                         void* stream) {
  const int cus = cu_count();
  if (!src || !dst || bytes == 0 || bytes % 16 ||
      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) || cus < 1 || blocks_per_cu < 1 ||
      blocks_per_cu > 64)
    return -1;
  const dim3 g(cus * blocks_per_cu), b(256);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  if (nt_store) hipLaunchKernelGGL(k_copy<true>, g, b, 0, static_cast<hipStream_t>(stream), s, d, (int64_t)(bytes / 16));
  else hipLaunchKernelGGL(k_copy<false>, g, b, 0, static_cast<hipStream_t>(stream), s, d, (int64_t)(bytes / 16));
  return status(hipGetLastError());
}

}  // extern "C"
