// Device-side MXFP4 helpers shared by the quantiser and attention kernels (gfx950).
//
// MXFP4 (Pith review of MXAttention, Axiom ledger axiom 1; 10100.com explainer):
// 32 E2M1 elements share one E8M0 power-of-two scale.  E2M1 rounding here is
// done by the gfx950 conversion v_cvt_scalef32_pk_fp4_f32, which rounds to
// nearest even, saturates to +-6, keeps the sign of values that round to zero,
// and divides by 2^(exponent of its scale operand) exactly before rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mxattn {

// E8M0 scale byte (shared exponent e plus the bias 127) for a block whose max
// magnitude has fp32 bit pattern `mbits` (finite, non-negative; zero and subnormals
// allowed).
//  CEIL(q): the smallest e with M <= q 2^e.  With M = 1.f 2^E and q = 1.g 2^qe,
//           that is E - qe when f <= g and E - qe + 1 otherwise.
//  OCP:     E - 2 (encoded as qe = 2 with a g that no f exceeds).
// e is clamped to [-127, 127], the byte to [0, 254].  Every M below 2^-126 (zero and
// subnormals included) needs e <= -127 under any rule with q >= 4, so reading E
// from the biased exponent field (E = -127 for those) and clamping is exact.
// Branch-free: adding 2^23 - 1 - g to the bits carries into the exponent field
// exactly when f > g, and the subtraction of qe is folded into the same constant
// (q <= 8, so the sum never overflows), leaving an add, a shift and a clamp.
__device__ __forceinline__ int mx_scale_byte(uint32_t mbits, Rule r) {
  const uint32_t carry = r.q_frac >= 0x7FFFFFu ? 0u : 0x7FFFFFu - r.q_frac;
  const int t = (int)(mbits + (carry - ((uint32_t)r.q_exp << 23)));
  const int eb = t >> 23;  // arithmetic shift: E + 127 - qe + (f > g), rounded down
  return eb < 0 ? 0 : (eb > 254 ? 254 : eb);
}

// The conversion's scale operand for scale byte eb: an fp32 whose exponent field is
// eb (the instruction uses only that field, as an E8M0 value; the field 0 stands for
// 2^-127 and subnormal inputs convert exactly).
__device__ __forceinline__ float e8m0_scale(int eb) { return __uint_as_float((uint32_t)eb << 23); }

// Two fp32 values -> one byte of two E2M1 codes (a in the low nibble) written
// into byte `SEL` of `old`, after dividing by 2^e (e from the scale operand).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_fp4(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Quantise 32 fp32 values v[0..31] with the conversion's scale operand s (an fp32 whose
// exponent field is the E8M0 byte) into 4 dwords of codes, element k in nibble k.
__device__ __forceinline__ void quant_pairs(const float* v, float s, uint32_t out[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // all four bytes of r are written below, so its initial value is irrelevant:
    // start from a value that is dead afterwards instead of materialising a zero
    uint32_t r = __float_as_uint(v[8 * w + 0]);
    r = cvt_pk_fp4<0>(r, v[8 * w + 0], v[8 * w + 1], s);
    r = cvt_pk_fp4<1>(r, v[8 * w + 2], v[8 * w + 3], s);
    r = cvt_pk_fp4<2>(r, v[8 * w + 4], v[8 * w + 5], s);
    r = cvt_pk_fp4<3>(r, v[8 * w + 6], v[8 * w + 7], s);
    out[w] = r;
  }
}

// The same with scale byte eb (any eb in [0, 254]).
__device__ __forceinline__ void quant32(const float* v, int eb, uint32_t out[4]) { quant_pairs(v, e8m0_scale(eb), out); }

// Largest |v[i]| of a 32-element block as fp32 bits, with the NaN-propagating
// maximum (v_maximum3_f32 with |.| operand modifiers): the result, sign cleared,
// is >= 0x7F800000 exactly when some element is not finite, and is otherwise the
// bit pattern of the largest magnitude.
__device__ __forceinline__ float amax2(float a, float b) {
  return __builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b));
}
__device__ __forceinline__ float amax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(amax2(a, b), __builtin_fabsf(c));
}
__device__ __forceinline__ uint32_t absmax32_bits(const float* v) {
  float u[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) u[i] = amax3(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
  u[10] = amax2(v[30], v[31]);
  const float w0 = amax3(u[0], u[1], u[2]), w1 = amax3(u[3], u[4], u[5]);
  const float w2 = amax3(u[6], u[7], u[8]), w3 = amax2(u[9], u[10]);
  return __float_as_uint(amax2(amax3(w0, w1, w2), w3)) & 0x7FFFFFFFu;
}

// Scale bytes written straight into the attention kernel's per-tile operand order (the
// layout of mxattn_arrange_scales, 512 bytes per 128-key tile and head), for the forward's
// own K^ and V^T.  K: the byte of key `key`, d-block b sits in dword 2 lane + b / 2, byte
// t, of tile key / 128, with lane = r + 32 (b % 2) and (t, r) the inverse of the kernel's
// key permutation kappa(t, r) = 64(t/2) + 32((r/4)%2) + 16(t%2) + 4(r/8) + r%4.
__device__ __forceinline__ int64_t arranged_k_offset(int64_t key, int b) {
  const int k = (int)(key & 127);
  const int t = 2 * (k >> 6) + ((k >> 4) & 1);
  const int r = 8 * ((k >> 2) & 3) + 4 * ((k >> 5) & 1) + (k & 3);
  return 512 * (key >> 7) + 4 * (2 * (r + 32 * (b & 1)) + (b >> 1)) + t;
}
// V^T: the byte of channel ch, 32-key block kb sits in dword 2 lane + (kb / 2) % 2, byte
// ch / 32, of tile kb / 4, with lane = ch % 32 + 32 (kb % 2).
__device__ __forceinline__ int64_t arranged_v_offset(int ch, int64_t kb) {
  return 512 * (kb >> 2) + 4 * (2 * ((ch & 31) + 32 * (int)(kb & 1)) + (int)((kb >> 1) & 1)) + (ch >> 5);
}
// (head, row within the head) of a global row, rows_per_head >= 1; 32-bit division when
// every row index fits (the common case: B H N < 2^31), 64-bit otherwise.
__device__ __forceinline__ void split_row(int64_t row, int64_t rows_per_head, int64_t nrows, int64_t& head,
                                          int64_t& r) {
  if (nrows < (int64_t(1) << 31)) {
    const uint32_t h = (uint32_t)row / (uint32_t)rows_per_head;
    head = h;
    r = (uint32_t)row - h * (uint32_t)rows_per_head;
  } else {
    head = row / rows_per_head;
    r = row - head * rows_per_head;
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Global->LDS DMA of 16, 4 or 2 bytes per lane through a raw buffer descriptor:
// lane L writes at lds + 16 L (the 4- and 2-byte forms at lds + 4 L, zero-extended);
// `lds` must be the same in every lane, and offsets past the descriptor's size read 0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
// Streaming form for data read exactly once (the quantisers' inputs): the load is marked
// non-temporal (cache-policy bit nt), which keeps it from displacing reused lines.
__device__ __forceinline__ void dma16_stream(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 2);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}
__device__ __forceinline__ void dma2(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 2, off, 0, 0, 0);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace mxattn
