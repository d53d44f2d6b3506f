// MXFP4 block quantisers for gfx950 (HBM-bound streaming kernels).
//
//  k_quant_hadamard : fused Hadamard-d rotation + block quantisation along the
//                     last axis (Q and K; the standalone quantise pass).
//  k_quant_last     : block quantisation along the last axis, no rotation.
//  k_quant_rows     : block quantisation down the rows (V along tokens), written
//                     transposed so each channel's kv codes are contiguous.
//
// Method: Pith review of MXAttention, Axiom ledger (axiom 1: 32-element E2M1
// blocks with one E8M0 scale; Hadamard rotation on Q/K, sec. 4.3) and Figure 3
// caption (scale rules); 10100.com explainer (rounding and saturation).
// The rotation is the fp32 fast Walsh-Hadamard transform with butterflies
// h = 1, 2, ..., d/2 followed by one multiply by fl32(1/sqrt d): every output is
// produced by the same sequence of IEEE fp32 adds/subs as that definition, so
// the codes are bit-identical to any implementation of it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "mx_device.h"

namespace mxattn {

// Non-finite marker and the block max of |x| taken on the fp32 bit patterns:
// for non-negative floats integer order is float order, and NaN/Inf patterns
// sort above every finite value, so max >= 0x7F800000 flags a non-finite block.
__device__ __forceinline__ uint32_t absbits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------
// Fused Hadamard + quantise.  D in {64, 128}; EB = bytes per input element (2 = bf16, 4 = fp32).
// One row is held by LPR = D/64 lanes, 64 elements each; a 256-thread block
// handles ROWS = 256/LPR rows.  The tile is read from HBM with fully coalesced
// 16-byte loads into LDS (rows padded by 16 bytes so that the per-lane row reads
// are bank-conflict free), then each lane reads its 64 elements.
// Butterflies h = 1..32 run inside the lane; for D = 128 the h = 64 stage pairs
// the two lanes of a row through a DPP quad permute (lanes 2r, 2r+1).
template <int D, int EB>
__global__ __launch_bounds__(256) void k_quant_hadamard(const uint8_t* __restrict__ x, int64_t nrows,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, Rule rule,
                                                        float c) {
  constexpr int LPR = D / 64;
  constexpr int ROWS = 256 / LPR;
  constexpr int ROW_BYTES = D * EB;
  constexpr int STRIDE = ROW_BYTES + 16;
  constexpr int CH_PER_ROW = ROW_BYTES / 16;
  constexpr int NCH = ROWS * CH_PER_ROW;  // 16-byte chunks in the tile
  __shared__ __attribute__((aligned(16))) uint8_t tile[ROWS * STRIDE];

  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS;
  const int64_t left = nrows - row0;
  const int nr = left < ROWS ? (int)left : ROWS;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row0 * ROW_BYTES);
  const int nch_valid = nr * CH_PER_ROW;
#pragma unroll
  for (int k = 0; k < NCH / 256; ++k) {
    const int ch = tid + 256 * k;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ch < nch_valid) {
      const u32x4 w = __builtin_nontemporal_load(src + ch);  // streamed once: do not keep in cache
      v = make_uint4(w.x, w.y, w.z, w.w);
    }
    const int r = ch / CH_PER_ROW, q = ch % CH_PER_ROW;
    *reinterpret_cast<uint4*>(tile + r * STRIDE + 16 * q) = v;
  }
  __syncthreads();

  const int lr = tid / LPR;     // row within the tile
  const int half = tid % LPR;   // which 64 elements of the row
  float v[64];
  {
    const uint8_t* p = tile + lr * STRIDE + half * 64 * EB;
    if constexpr (EB == 2) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint4 w = *reinterpret_cast<const uint4*>(p + 16 * q);
        v[8 * q + 0] = bf16lo(w.x); v[8 * q + 1] = bf16hi(w.x);
        v[8 * q + 2] = bf16lo(w.y); v[8 * q + 3] = bf16hi(w.y);
        v[8 * q + 4] = bf16lo(w.z); v[8 * q + 5] = bf16hi(w.z);
        v[8 * q + 6] = bf16lo(w.w); v[8 * q + 7] = bf16hi(w.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float4 w = *reinterpret_cast<const float4*>(p + 16 * q);
        v[4 * q + 0] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
      }
    }
  }
  // in-lane butterflies h = 1, 2, 4, 8, 16, 32 (element index bits 0..5)
#pragma unroll
  for (int h = 1; h < 64; h *= 2) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  if constexpr (LPR == 2) {
    // h = 64: lane 2r holds elements 0..63 (the "a" side), lane 2r+1 holds 64..127.
    // a-lane: own + partner = a + b;  b-lane: partner + (-own) = a - b.
    const uint32_t sgn = (uint32_t)half << 31;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), 0xB1, 0xF, 0xF, false));
      v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ sgn);
    }
  }

  const int64_t grow = row0 + lr;
  if (lr >= nr) return;
  uint8_t* crow = codes + grow * (D / 2) + half * 32;
  uint8_t* srow = scales + grow * (D / 32) + half * 2;
  uint8_t sb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float* blk = v + 32 * b;
    // integer max of |bits|: NaN and Inf sort above every finite value
    uint32_t mh = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) mh = max(mh, absbits(blk[i]));
#pragma unroll
    for (int i = 0; i < 32; ++i) blk[i] = blk[i] * c;
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    if (mh >= 0x7F800000u) {
      sb[b] = 0xFF;
    } else {
      // max |fl(v c)| = fl(max|v| c), since rounding is monotone
      const uint32_t mb = __float_as_uint(__uint_as_float(mh) * c);
      const int e = mx_exponent(mb, rule);
      quant32(blk, e, q);
      sb[b] = (uint8_t)(e + 127);
    }
    *reinterpret_cast<uint4*>(crow + 16 * b) = make_uint4(q[0], q[1], q[2], q[3]);
  }
  *reinterpret_cast<uint16_t*>(srow) = (uint16_t)(sb[0] | (sb[1] << 8));
}

// ---------------------------------------------------------------------------
// Plain quantise along the last axis: one thread per 32-element block.
template <int EB>
__global__ __launch_bounds__(256) void k_quant_last(const uint8_t* __restrict__ x, int64_t nblocks,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, Rule rule) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  float v[32];
  const uint4* src = reinterpret_cast<const uint4*>(x + blk * 32 * EB);
  if constexpr (EB == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 w = src[q];
      v[8 * q + 0] = bf16lo(w.x); v[8 * q + 1] = bf16hi(w.x);
      v[8 * q + 2] = bf16lo(w.y); v[8 * q + 3] = bf16hi(w.y);
      v[8 * q + 4] = bf16lo(w.z); v[8 * q + 5] = bf16hi(w.z);
      v[8 * q + 6] = bf16lo(w.w); v[8 * q + 7] = bf16hi(w.w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint4 w = src[q];
      v[4 * q + 0] = __uint_as_float(w.x); v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z); v[4 * q + 3] = __uint_as_float(w.w);
    }
  }
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) mb = max(mb, absbits(v[i]));
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  uint8_t sb;
  if (mb >= 0x7F800000u) {
    sb = 0xFF;
  } else {
    const int e = mx_exponent(mb, rule);
    quant32(v, e, q);
    sb = (uint8_t)(e + 127);
  }
  *reinterpret_cast<uint4*>(codes + blk * 16) = make_uint4(q[0], q[1], q[2], q[3]);
  scales[blk] = sb;
}

// ---------------------------------------------------------------------------
// Quantise down the rows (tokens) and write transposed:
//   x [batch, rows, cols] -> codes [batch, cols, P/2], scales [batch, cols, P/32].
// A 256-thread block owns a tile of 128 tokens x 128 columns.  The tile is read
// with coalesced dword loads into LDS (zero where rows >= `rows` or cols >=
// `cols`), then thread t quantises columns (2p, 2p+1), p = t % 64, over the 32
// tokens of block t / 64.  blockIdx.x: token tile; blockIdx.y: column tile;
// blockIdx.z: batch.
template <int EB>
__global__ __launch_bounds__(256) void k_quant_rows(const uint8_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t P,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, Rule rule) {
  constexpr int TT = 128;                 // tokens per tile
  constexpr int TC = 128;                 // columns per tile
  constexpr int RB = TC * EB;             // bytes of one tile row
  constexpr int STRIDE = RB + 4;          // dword padding
  __shared__ __attribute__((aligned(16))) uint8_t tile[TT * STRIDE];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int64_t c0 = (int64_t)blockIdx.y * TC;
  const int64_t b = blockIdx.z;
  const uint8_t* xb = x + b * rows * cols * EB;
  // load: the tile is TT rows of RB bytes = TT * RB / 4 dwords
  constexpr int NDW = TT * RB / 4;
  constexpr int DW_PER_ROW = RB / 4;
  const int64_t cbytes_valid = (cols - c0) * EB;  // bytes of valid columns in this tile row
#pragma unroll 4
  for (int k = tid; k < NDW; k += 256) {
    const int r = k / DW_PER_ROW, q = k % DW_PER_ROW;
    const int64_t tok = t0 + r;
    uint32_t w = 0;
    if (tok < rows && 4 * q < cbytes_valid)
      w = *reinterpret_cast<const uint32_t*>(xb + (tok * cols + c0) * EB + 4 * q);
    *reinterpret_cast<uint32_t*>(tile + r * STRIDE + 4 * q) = w;
  }
  __syncthreads();
  const int p = tid % 64, blk = tid / 64;
  float va[32], vb[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint8_t* rp = tile + (32 * blk + k) * STRIDE + 2 * p * EB;
    if constexpr (EB == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(rp);
      va[k] = bf16lo(w);
      vb[k] = bf16hi(w);
    } else {
      uint2 w = *reinterpret_cast<const uint2*>(rp);
      va[k] = __uint_as_float(w.x);
      vb[k] = __uint_as_float(w.y);
    }
  }
  const int64_t col = c0 + 2 * p;
  const int64_t kv0 = t0 + 32 * blk;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* v = s ? vb : va;
    if (col + s >= cols) break;
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) mb = max(mb, absbits(v[i]));
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    uint8_t sb;
    if (mb >= 0x7F800000u) {
      sb = 0xFF;
    } else {
      const int e = mx_exponent(mb, rule);
      quant32(v, e, q);
      sb = (uint8_t)(e + 127);
    }
    const int64_t crow = b * cols + col + s;
    *reinterpret_cast<uint4*>(codes + crow * (P / 2) + kv0 / 2) = make_uint4(q[0], q[1], q[2], q[3]);
    scales[crow * (P / 32) + kv0 / 32] = sb;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_quant_hadamard(const void* x, int eb, int d, int64_t nrows, uint8_t* codes,
                                 uint8_t* scales, Rule rule, float c, hipStream_t s) {
  const int rows_per_block = 256 / (d / 64);
  const int64_t grid = (nrows + rows_per_block - 1) / rows_per_block;
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  if (d == 128 && eb == 2)
    hipLaunchKernelGGL((k_quant_hadamard<128, 2>), dim3((unsigned)grid), dim3(256), 0, s, xp, nrows, codes, scales, rule, c);
  else if (d == 128 && eb == 4)
    hipLaunchKernelGGL((k_quant_hadamard<128, 4>), dim3((unsigned)grid), dim3(256), 0, s, xp, nrows, codes, scales, rule, c);
  else if (d == 64 && eb == 2)
    hipLaunchKernelGGL((k_quant_hadamard<64, 2>), dim3((unsigned)grid), dim3(256), 0, s, xp, nrows, codes, scales, rule, c);
  else if (d == 64 && eb == 4)
    hipLaunchKernelGGL((k_quant_hadamard<64, 4>), dim3((unsigned)grid), dim3(256), 0, s, xp, nrows, codes, scales, rule, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_last(const void* x, int eb, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                             Rule rule, hipStream_t s) {
  const int64_t grid = (nblocks + 255) / 256;
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  if (eb == 2)
    hipLaunchKernelGGL((k_quant_last<2>), dim3((unsigned)grid), dim3(256), 0, s, xp, nblocks, codes, scales, rule);
  else
    hipLaunchKernelGGL((k_quant_last<4>), dim3((unsigned)grid), dim3(256), 0, s, xp, nblocks, codes, scales, rule);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int eb, int64_t batch, int64_t rows, int64_t cols,
                             int64_t P, uint8_t* codes, uint8_t* scales, Rule rule, hipStream_t s) {
  dim3 grid((unsigned)(P / 128), (unsigned)((cols + 127) / 128), (unsigned)batch);
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  if (eb == 2)
    hipLaunchKernelGGL((k_quant_rows<2>), grid, dim3(256), 0, s, xp, rows, cols, P, codes, scales, rule);
  else
    hipLaunchKernelGGL((k_quant_rows<4>), grid, dim3(256), 0, s, xp, rows, cols, P, codes, scales, rule);
  return hipGetLastError();
}

}  // namespace mxattn
