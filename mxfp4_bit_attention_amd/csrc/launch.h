// Host-side launchers of the HIP kernels (internal to libmxattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn {

// Shared-scale rule in the form the kernels use: for a block max M = 1.f * 2^E the
// shared exponent is e = E - q_exp + (f > q_frac), f and q_frac being 23-bit
// fractions.  CEIL(q) with q = 1.g * 2^q_exp (UOS is CEIL(7.25)) sets q_frac = g;
// the OCP floor rule e = floor(log2 M) - 2 sets q_exp = 2 and a q_frac no fraction
// exceeds, so one branch-free formula serves every rule.
struct Rule {
  int q_exp;
  uint32_t q_frac;
};

// Quantisers.  With err == nullptr they store codes and scales; with err != nullptr
// they store nothing and add {sum (x - dequant)^2, sum x^2, non-finite blocks} to err[0..2].
// Scales go to the layout of mxattn_quantize, or -- arr_keys > 0 / arranged, for the
// forward's own K^ and V^T -- straight into the attention kernel's per-tile operand order
// (the layout of mxattn_arrange_scales: arr_keys rows per head, 4 arr_pad bytes per head;
// for V one head per batch item and 4 P bytes).  The arranged bytes of key slots past the
// last key of a head are not written: the attention kernel masks those keys' logits.
// Fused Hadamard + quantise along the last axis; d in {64, 128}; eb = 2 (bf16) or 4 (fp32).
hipError_t launch_quant_hadamard(const void* x, int eb, int d, int64_t nrows, uint8_t* codes,
                                 uint8_t* scales, Rule rule, float c, double* err, hipStream_t s,
                                 int64_t arr_keys = 0, int64_t arr_pad = 0);
// Quantise along the last axis in 32-element blocks (nblocks blocks, contiguous;
// blocks_per_row of them per row when the scales are arranged).
hipError_t launch_quant_last(const void* x, int eb, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                             Rule rule, double* err, hipStream_t s, int blocks_per_row = 0, int64_t arr_keys = 0,
                             int64_t arr_pad = 0);
// Quantise down the rows, transposed output with P (multiple of 128) padded tokens.
hipError_t launch_quant_rows(const void* x, int eb, int64_t batch, int64_t rows, int64_t cols,
                             int64_t P, uint8_t* codes, uint8_t* scales, Rule rule, double* err, hipStream_t s,
                             bool arranged = false);
// The forward's K and V in one launch: the Hadamard quantiser over K [heads, nkv, d] and the
// token-axis quantiser over V [heads, nkv, d], both with arranged scales (P padded tokens).
hipError_t launch_quant_kv(const void* k, const void* v, int eb, int d, int64_t heads, int64_t nkv, int64_t P,
                          uint8_t* kc, uint8_t* ksa, uint8_t* vc, uint8_t* vsa, Rule rule, float c, hipStream_t s);
// Sets n doubles to zero with a kernel (graph-capturable, unlike a memset node).
hipError_t launch_zero_f64(double* p, int n, hipStream_t s);

struct AttnArgs {
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  // Optional pre-arranged K^ and V^T scales (launch_arrange_scales); when set, ks and
  // vs are unused.  512 bytes per kv tile per head, each.
  const uint8_t* ksa;
  const uint8_t* vsa;
  void* o;
  uint8_t* pc;   // optional P^ dump
  uint8_t* ps;
  int64_t heads;  // B * H
  int64_t nq;
  int64_t nkv;
  int64_t kv_pad;  // P: padded tokens of the transposed V layout
  float scale_log2;  // softmax_scale * log2(e)
  int out_bf16;
  // Unquantised Q [heads, nq, d] (bf16 or fp32): when set, the kernel rotates and
  // quantises its own query rows in its prologue (with the P~ rule) and qc/qs are unused.
  const void* qraw;
  int q_bf16;
  int q_hadamard;
  float q_c;  // fl32(1/sqrt(d)), the rotation's final multiplier
  // The P~ rule in the attention kernel's log-domain form: the OCP floor rule
  // (p_floor = 1), or CEIL(q) with p_log2q = fl32(log2 q).
  int p_floor;
  float p_log2q;
};

hipError_t launch_attention(const AttnArgs& a, int d, int pnq, Rule p_rule, hipStream_t s);
// Re-orders the scales of K^ [heads, nkv, d/32] and V^T [heads, d, kv_pad/32] into the
// per-tile order the attention kernel's lanes use (heads * kv_pad * 4 bytes each).
hipError_t launch_arrange_scales(const uint8_t* ks, const uint8_t* vs, int64_t heads, int64_t nkv, int64_t kv_pad,
                                 int d, uint8_t* ksa, uint8_t* vsa, hipStream_t s);

constexpr int kKvTile = 128;

// The argument checks of mxattn_forward other than those of its workspace, with `who`
// naming the entry point in the error message; on success *workspace_bytes is the
// workspace the call needs.  Returns MXATTN_OK or the negative status (message set).
int forward_arg_check(const void* Q, const void* K, const void* V, int32_t dtype, int64_t B, int64_t H, int64_t Nq,
                      int64_t Nkv, int64_t d, float softmax_scale, int32_t rule_kind, float qmax, const void* O,
                      const char* who, size_t* workspace_bytes);
// Sets the thread's mxattn_last_error() message; returns `status`.
int set_error(int status, const char* message);

}  // namespace mxattn
