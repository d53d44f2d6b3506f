// Fused MXFP4 attention forward with Pre-Normalization Quantization (gfx950).
//
// Method (Pith review of MXAttention, Figure 4 caption and Core claim; abstract;
// 10100.com explainer): FlashAttention-2 online softmax where the unnormalised
// exponential tile P~ = exp(S - m') is quantised to MXFP4 once, and that one
// quantised tile P^ feeds both the row-sum update and the P^ V update, so the
// normalised weights sum to one by construction.  With PNQ off the row sum
// uses the unquantised P~ (the direct placement of Figure 4(C)).
//
// Both products are block-scaled 32x32x64 MFMAs (v_mfma_scale_f32_32x32x64_f8f6f4
// with fp4 operands and E8M0 scales), computed transposed so that every lane owns
// one query and two aligned 32-key blocks of each 128-key tile.  Lane (i, h)
// (i = lane % 32, h = lane / 32):
//   S^T = K^ Q^^T  : MFMA (t, s), t = 0..3, s = 0..d/64-1: A = 32 keys x 64 d (LDS),
//                    B = Q^ (registers, query i, d-block 2s + h).  Row rho of MFMA t
//                    is key kappa(t, rho), chosen so that output element v of lane
//                    (i, h) is key 64(t/2) + 32h + 16(t%2) + v of query i: after the
//                    four MFMAs the lane holds keys 64c + 32h + 0..31 (c = 0, 1).
//   O^T += V^^T P^^T : MFMA (ct, c): A = 32 channels x 64 keys (LDS), B = P^ of the
//                    64-key chunk c, which is exactly the lane's block c quantised
//                    in registers with its E8M0 byte, so P^ never leaves registers.
// The row max needs one cross-lane step (v_permlane32_swap); the PNQ row sum is one
// extra MFMA per chunk against an all-ones A operand, which sums the same P^ codes
// the P^ V product uses.  A 32x32x64 MFMA leaves the vector ALU free for part of
// its duration (the 16x16x128 form does not), so ALU work placed beside these
// MFMAs, in this wave or in the other waves of the SIMD, runs in their shadow.
// The MFMAs' E8M0 scale operands come either pre-arranged per tile in the lanes'
// operand order (as the forward's quantisers write them, or k_arrange_scales; one
// 8-byte LDS read per lane and tile) or in the quantiser's layout, from which each lane
// gathers its bytes with v_perm.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mxattn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// D = A * B + C with fp4 A and B, E8M0 scales chosen by byte OPA of sa / byte 0 of sb.
template <int OPA>
__device__ __forceinline__ v16f mma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, OPA, sa, 0, sb);
}

// NaN-propagating maxima (v_maximum_f32 / v_maximum3_f32): a NaN logit -- which the
// block-scaled MFMA produces for every product with a block whose E8M0 scale is 0xFF,
// the quantisers' mark of a block that held Inf or NaN -- makes the row max NaN, so
// alpha, l and the row's output become NaN as IEEE arithmetic on the dequantised
// operands would make them.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// max / sum over lanes l and l ^ 32
__device__ __forceinline__ float xmax2(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xsum2(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int BC = kKvTile;  // 128 keys per kv tile
// A workgroup is 4 waves (one per SIMD) of 32 queries each, and three workgroups share
// a CU (at most 168 VGPRs per wave, 3 x 52 KB of LDS): each SIMD then runs one wave of
// each, and since the workgroups synchronise on separate barriers they drift out of
// phase, so one wave's softmax runs beside another's MFMAs.
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup
constexpr int BR = 32 * NW;  // queries per workgroup

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding: vmcnt low
// bits [3:0] and high bits [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define MX_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))

// One kv tile in LDS.  Every region is filled by global->LDS DMA, where lane L of a
// wave writes 16 (or 4) bytes at base + 16 L (or 4 L); the layouts below are chosen
// so that each MFMA fragment is one contiguous 1 KB read per wave.
//  K codes  [t][s][l] 16-byte units: unit (t, s, l) = d-block 2s + l/32 of key kappa(t, l%32)
//  K scales [4 i + t] dwords: the d/32 scale bytes of key kappa(t, i)
//  V codes  [ct][c][l]: unit (ct, c, l) = keys 64c + 32(l/32) .. +31 of channel 32ct + l%32
//  V scales [NCT i + ct] dwords: the 4 scale bytes (one per 32-key block) of channel 32ct + i
// or, when the scales come pre-arranged (the forward's own workspace, written in that
// order by its quantisers; mxattn_arrange_scales for caller-quantised operands), the two
// scale regions hold exactly the lanes' MFMA scale operands:
//  K scales [2 lane + s] dwords: byte t = scale of key kappa(t, lane%32), d-block 2s + lane/32
//  V scales [2 lane + c] dwords: byte ct = scale of channel 32ct + lane%32, key block 2c + lane/32
// so a lane loads its operands with one 8-byte read and no byte gathers.
template <int D>
struct Geo {
  static constexpr int S = D / 64;     // d-steps of an S^T MFMA
  static constexpr int NCT = D / 32;   // 32-channel tiles of O
  static constexpr int KC = BC * D / 2;
  static constexpr int KS = 4 * BC;
  static constexpr int VC = D * BC / 2;
  static constexpr int VS = 4 * BC;  // the larger of 4 D (gathered) and 512 (pre-arranged)
  static constexpr int OFF_KS = KC;
  static constexpr int OFF_VC = KC + KS;
  static constexpr int OFF_VS = KC + KS + VC;
  static constexpr int STAGE = KC + KS + VC + VS;
  static constexpr int CODE_DMA = D / 64;        // 1 KB code loads per wave per tile, for K and for V
  static constexpr int NDMA = 2 * CODE_DMA + 1;  // DMA instructions per wave per tile
  static_assert(KC == NW * CODE_DMA * 1024 && VC == NW * CODE_DMA * 1024, "code DMA split");
};

// Key of row rho of S^T MFMA t: output element v of lane (i, h) is row
// 8(v/4) + 4h + v%4, which this maps to key 64(t/2) + 32h + 16(t%2) + v.
__device__ __forceinline__ int kappa(int t, int rho) {
  return 64 * (t >> 1) + 32 * ((rho >> 2) & 1) + 16 * (t & 1) + 4 * (rho >> 3) + (rho & 3);
}

// Per-lane byte offsets of a wave's tile DMAs (the same for every tile).
template <int D>
struct DmaOffsets {
  uint32_t k[Geo<D>::CODE_DMA];
  uint32_t v[Geo<D>::CODE_DMA];
  uint32_t s;  // waves 0-1: key scales; waves 2-3: channel scales
};

template <int D, bool PRE>
__device__ __forceinline__ DmaOffsets<D> dma_offsets(int64_t kv_pad, int wave, int lane) {
  using G = Geo<D>;
  DmaOffsets<D> o;
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) {
    const int p = 64 * (G::CODE_DMA * wave + u) + lane;  // 16-byte unit of the K region
    const int t = p / (64 * G::S), s = (p / 64) % G::S, l = p % 64;
    o.k[u] = (uint32_t)(kappa(t, l & 31) * (D / 2) + 16 * (2 * s + (l >> 5)));
  }
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) {
    const int p = 64 * (G::CODE_DMA * wave + u) + lane;  // 16-byte unit of the V region
    const int ct = p / 128, c = (p / 64) % 2, l = p % 64;
    o.v[u] = (uint32_t)((32 * ct + (l & 31)) * (kv_pad / 2) + 32 * c + 16 * (l >> 5));
  }
  if constexpr (PRE) {
    o.s = (uint32_t)(4 * (64 * (wave & 1) + lane));  // 512 contiguous bytes per tile, K or V
  } else if (wave < 2) {
    const int p = 64 * wave + lane;  // dword 4 i + t of the K scale region
    o.s = (uint32_t)(kappa(p % 4, p / 4) * (D / 32));
  } else {
    const int p = (wave - 2) * (D / 2) + lane;  // dword NCT i + ct of the V scale region
    const int ch = 32 * (p % G::NCT) + p / G::NCT;
    o.s = (uint32_t)(ch * (kv_pad / 32));
  }
  return o;
}

// Raw buffer descriptor over `bytes` bytes from `base`; loads at offsets >= bytes
// return zero without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

// One head's tile sources and their sizes in bytes (below 2^31: at most 2^24 tokens).
struct TileSrc {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int kc_bytes, ks_bytes, vc_bytes, vs_bytes;
};

// Issue the DMAs of tile j into stage `st`: NDMA instructions per wave.  The buffer
// descriptors are rebuilt per tile on the scalar unit (base at the tile, size = bytes
// left), so keys past the last one, and whole tiles past the end, read as zero
// without touching memory.  Past the end the V^ descriptors still cover the head's
// other channels: those reads stay inside the head's V^ and are never used.
template <int D, bool PRE>
__device__ __forceinline__ void tile_dma(uint8_t* st, const DmaOffsets<D>& o, const TileSrc& src, int j, int wave,
                                         int lane) {
  using G = Geo<D>;
  const int kc0 = j * (BC * D / 2), ks0 = j * (BC * D / 32);
  const __amdgpu_buffer_rsrc_t rk = rsrc(src.kc + kc0, max(src.kc_bytes - kc0, 0));
  const __amdgpu_buffer_rsrc_t rv = rsrc(src.vc + 64 * j, src.vc_bytes - 64 * j);
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) dma16(rk, st + 1024 * (G::CODE_DMA * wave + u), o.k[u]);
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) dma16(rv, st + G::OFF_VC + 1024 * (G::CODE_DMA * wave + u), o.v[u]);
  if constexpr (PRE) {
    const int so = 512 * j;
    if (wave < 2) dma4(rsrc(src.ks + so, max(src.ks_bytes - so, 0)), st + G::OFF_KS + 256 * wave, o.s);
    else dma4(rsrc(src.vs + so, max(src.vs_bytes - so, 0)), st + G::OFF_VS + 256 * (wave - 2), o.s);
  } else if (wave < 2) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(src.ks + ks0, max(src.ks_bytes - ks0, 0));
    // a key's scales are one dword at D = 128, two bytes at D = 64
    if constexpr (D == 128) dma4(rs, st + G::OFF_KS + 256 * wave, o.s);
    else dma2(rs, st + G::OFF_KS + 256 * wave, o.s);
  } else if (lane < D / 2) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(src.vs + 4 * j, src.vs_bytes - 4 * j);
    dma4(rs, st + G::OFF_VS + 2 * D * (wave - 2), o.s);
  }
}

// v_perm selectors that gather byte b of two dwords into bytes 0-1 (lo) or 2-3 (hi).
struct Sel {
  uint32_t lo, hi;
};
__device__ __forceinline__ Sel byte_sel(uint32_t b) {
  return Sel{b | ((b + 4) << 8) | 0x0C0C0000u, 0x00000C0Cu | (b << 16) | ((b + 4) << 24)};
}
// Gather byte b of each of four dwords (x, y, z, w) into one dword, x in byte 0.
__device__ __forceinline__ uint32_t gather4(const u32x4& d, Sel s) {
  return __builtin_amdgcn_perm(d.y, d.x, s.lo) | __builtin_amdgcn_perm(d.w, d.z, s.hi);
}

// Workgroup barrier that the compiler may not move memory accesses across, without
// the memory wait that __syncthreads() adds (the DMA of the next tiles stays in flight).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Max of the 32 values of one block (a = keys 0..15, b = keys 16..31) with a max3 tree.
__device__ __forceinline__ float max32(const v16f& a, const v16f& b) {
  auto x = [&](int k) { return k < 16 ? a[k] : b[k - 16]; };
  float u[10];  // 16 max operations in three levels: 10, 4 and 2
#pragma unroll
  for (int i = 0; i < 10; ++i) u[i] = vmax3(x(3 * i), x(3 * i + 1), x(3 * i + 2));
  const float w0 = vmax3(u[0], u[1], u[2]), w1 = vmax3(u[3], u[4], u[5]);
  const float w2 = vmax3(u[6], u[7], u[8]), w3 = vmax3(u[9], x(30), x(31));
  return vmax(vmax3(w0, w1, w2), w3);
}

// Make the compiler produce these values at this point of the program (and not sink
// the instructions that produce them into a later branch).
template <int N>
__device__ __forceinline__ void pin_all(v16f (&x)[N], float& l) {
  if constexpr (N == 4) asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(l));
  else asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(l));
}

// Interleave the next N MFMAs of the scheduling region with K ALU/transcendental
// instructions each.
template <int N, int K>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, K, 0);  // K VALU / TRANS
  }
}

// Scale operand 2^e of the fp4 conversion for one P~ block, from y: the log2 of the
// block's largest P~ minus log2 q under CEIL(q) (the smallest e with max P~ <= q 2^e is
// ceil(y)), or that log2 itself under the OCP floor rule (e = floor(y) - 2).  Deciding in
// the log domain takes no exponential; it agrees with the decision on the fp32 value of
// max P~ except within a few fp32 ulps of a boundary.  v_ldexp_f32 makes 2^e subnormal or
// zero for e < -126, whose exponent field 0 is the E8M0 byte that clamps every e <= -127
// (the conversion reads only that field, as 2^-127).
template <bool PFLOOR>
__device__ __forceinline__ float p_block_scale(float y) {
  const float t = PFLOOR ? __builtin_floorf(y) : __builtin_ceilf(y);
  int e;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(e) : "v"(t));  // saturating: -inf -> INT_MIN, NaN -> 0
  return __builtin_amdgcn_ldexpf(PFLOOR ? 0.25f : 1.0f, e);
}

// P~ = exp2(x) of block c (x[2c], x[2c+1]) and its PNQ quantisation: codes pc, scale byte psc.
// y is the block's scale argument (p_block_scale); in the block that holds the row max the
// largest P~ is exactly 1 and y is exactly -log2 q (CEIL) or 0 (OCP).
// In a row whose running max is NaN the block's P~ are NaN; the P^ dump then records such a
// block as the quantiser records a non-finite block (scale 0xFF, codes 0), and that scale
// keeps the block's MFMAs NaN.  Without the dump the row's l is NaN anyway.
template <bool PNQ, bool DUMP, bool PFLOOR>
__device__ __forceinline__ void soft_exp(const v16f& xa, const v16f& xb, float y, uint32_t (&pc)[4], int& psc,
                                         float& ls) {
  float p[32];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    p[k] = __builtin_amdgcn_exp2f(xa[k]);
    p[16 + k] = __builtin_amdgcn_exp2f(xb[k]);
  }
  const float sc = p_block_scale<PFLOOR>(y);
  psc = (int)(__float_as_uint(sc) >> 23);
  quant_pairs(p, sc, pc);
  if constexpr (DUMP) {
    if (__builtin_isnan(y)) {
      psc = 0xFF;
      pc[0] = pc[1] = pc[2] = pc[3] = 0u;
    }
  }
  if constexpr (!PNQ) {
#pragma unroll
    for (int k = 0; k < 32; ++k) ls += p[k];
  }
}

// O~^T += V^^T P^^T for the 64-key chunk c (its V^ fragments read here, so only one
// chunk's occupy registers), plus with PNQ the row sum of the same P^: r = its total.
template <int D, bool PNQ>
__device__ __forceinline__ void pv_chunk(v16f (&acc)[D / 32], const uint8_t* __restrict__ st, int lane, int vsw,
                                         int c, const v8i& ones, const uint32_t (&pc)[4], int psc, float& r) {
  using G = Geo<D>;
  constexpr int NCT = D / 32;
  v8i vf[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(st + G::OFF_VC + 1024 * (2 * ct + c) + 16 * lane);
    vf[ct] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  }
  const v8i pf = v8i{(int)pc[0], (int)pc[1], (int)pc[2], (int)pc[3], 0, 0, 0, 0};
  if constexpr (PNQ) r = mma<0>(ones, pf, v16f{}, 127, psc)[0];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (ct == 0) acc[ct] = mma<0>(vf[ct], pf, acc[ct], vsw, psc);
    if (ct == 1) acc[ct] = mma<1>(vf[ct], pf, acc[ct], vsw, psc);
    if (ct == 2) acc[ct] = mma<2>(vf[ct], pf, acc[ct], vsw, psc);
    if (ct == 3) acc[ct] = mma<3>(vf[ct], pf, acc[ct], vsw, psc);
  }
}

// One kv tile for one wave's 32 queries.  `rem` (TAIL only) is the number of valid
// keys in the tile.
template <int D, bool PRE, bool PNQ, bool DUMP, bool PFLOOR, bool TAIL>
__device__ __forceinline__ void attend_tile(const uint8_t* __restrict__ st, int lane, Sel sel0, Sel sel1, int rem,
                                            const v8i (&qf)[D / 64], const int (&qsc)[D / 64],
                                            v16f (&acc)[D / 32], float& m, float& l, float cl, float plq,
                                            const AttnArgs& a, int64_t qrow, int64_t head, int j,
                                            const uint32_t* lones) {
  using G = Geo<D>;
  constexpr int S = G::S;
  constexpr int NCT = G::NCT;
  const int i = lane & 31;
  const int h = lane >> 5;

  // K^ scales: MFMA (t, s) uses keys kappa(t, .), d-block 2s + h
  int ksw[S];
  if constexpr (PRE) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(st + G::OFF_KS + 8 * lane);
    ksw[0] = (int)d.x;
    if constexpr (S == 2) ksw[1] = (int)d.y;
  } else {
    const u32x4 d = *reinterpret_cast<const u32x4*>(st + G::OFF_KS + 16 * i);
    ksw[0] = (int)gather4(d, sel0);
    if constexpr (S == 2) ksw[1] = (int)gather4(d, sel1);
  }
  const v16f z = {};
  v16f x[4];
  // K^ fragments read in two halves (keys of chunk 0, then chunk 1), each just before
  // its MFMAs, so that only half of them occupy registers at a time
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    v8i kf[2][S];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(st + 1024 * (S * (2 * c + tt) + s) + 16 * lane);
        kf[tt][s] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      }
    if (c == 0) {
      x[0] = mma<0>(kf[0][0], qf[0], z, ksw[0], qsc[0]);
      x[1] = mma<1>(kf[1][0], qf[0], z, ksw[0], qsc[0]);
      if constexpr (S == 2) {
        x[0] = mma<0>(kf[0][1], qf[1], x[0], ksw[1], qsc[1]);
        x[1] = mma<1>(kf[1][1], qf[1], x[1], ksw[1], qsc[1]);
      }
    } else {
      x[2] = mma<2>(kf[0][0], qf[0], z, ksw[0], qsc[0]);
      x[3] = mma<3>(kf[1][0], qf[0], z, ksw[0], qsc[0]);
      if constexpr (S == 2) {
        x[2] = mma<2>(kf[0][1], qf[1], x[2], ksw[1], qsc[1]);
        x[3] = mma<3>(kf[1][1], qf[1], x[3], ksw[1], qsc[1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (TAIL) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int lim = rem - 64 * (t >> 1) - 32 * h - 16 * (t & 1);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (v >= lim) x[t][v] = -INFINITY;
    }
  }
  const float bm0 = max32(x[0], x[1]);
  const float bm1 = max32(x[2], x[3]);
  const float mnew = vmax(m, xmax2(vmax(bm0, bm1)));
  const float alpha = __builtin_amdgcn_exp2f((m - mnew) * cl);
  m = mnew;
  const float mc = mnew * cl;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) x[t][v] = __builtin_fmaf(x[t][v], cl, -mc);
  // the blocks' scale arguments from a difference first: exactly 0 in the block that
  // holds the row max, whose P~ block max is then exactly 1 as the method defines it (an
  // fma of bm alone can leave a rounding residue and move the exponent)
  const float y0 = PFLOOR ? (bm0 - mnew) * cl : __builtin_fmaf(bm0 - mnew, cl, -plq);
  const float y1 = PFLOOR ? (bm1 - mnew) * cl : __builtin_fmaf(bm1 - mnew, cl, -plq);

  // V^ scales (the fragments are read per chunk in pv_chunk)
  int vsw[2];
  if constexpr (PRE) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(st + G::OFF_VS + 8 * lane);
    vsw[0] = (int)d.x;
    vsw[1] = (int)d.y;
  } else if constexpr (NCT == 4) {
    const u32x4 d = *reinterpret_cast<const u32x4*>(st + G::OFF_VS + 16 * i);
    vsw[0] = (int)gather4(d, sel0);
    vsw[1] = (int)gather4(d, sel1);
  } else {
    const u32x2 d = *reinterpret_cast<const u32x2*>(st + G::OFF_VS + 8 * i);
    vsw[0] = (int)__builtin_amdgcn_perm(d.y, d.x, sel0.lo);
    vsw[1] = (int)__builtin_amdgcn_perm(d.y, d.x, sel1.lo);
  }
  v8i ones;
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(lones);
    ones = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  }

  uint32_t pc0[4], pc1[4];
  int psc0, psc1;
  float ls = 0.0f;
  soft_exp<PNQ, DUMP, PFLOOR>(x[0], x[1], y0, pc0, psc0, ls);

  // rescale the running state when any row's max moved (alpha == 1 is exact)
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] *= alpha;
  }
  __builtin_amdgcn_sched_barrier(0);
  float r0 = 0.0f, r1 = 0.0f;
  pv_chunk<D, PNQ>(acc, st, lane, vsw[0], 0, ones, pc0, psc0, r0);
  soft_exp<PNQ, DUMP, PFLOOR>(x[2], x[3], y1, pc1, psc1, ls);
  interleave_mfma<NCT + (PNQ ? 1 : 0), 6>();
  __builtin_amdgcn_sched_barrier(0);
  pv_chunk<D, PNQ>(acc, st, lane, vsw[1], 1, ones, pc1, psc1, r1);
  if constexpr (PNQ) l = __builtin_fmaf(l, alpha, r0 + r1);
  else l = __builtin_fmaf(l, alpha, xsum2(ls));

  if constexpr (DUMP) {
    if (qrow < a.nq) {
      const int64_t prow = head * a.nq + qrow;
      const uint32_t* pcs[2] = {pc0, pc1};
      const int pscs[2] = {psc0, psc1};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t key0 = (int64_t)j * BC + 64 * c + 32 * h;
        *reinterpret_cast<uint4*>(a.pc + prow * (a.kv_pad / 2) + key0 / 2) =
            make_uint4(pcs[c][0], pcs[c][1], pcs[c][2], pcs[c][3]);
        a.ps[prow * (a.kv_pad / 32) + key0 / 32] = (uint8_t)pscs[c];
      }
    }
  }
}

// Fused Q quantisation (mxattn_forward): lane (i, h) turns elements 32(2s + h) ..
// +31, s = 0..d/64-1, of query row `row` into MXFP4 blocks exactly as the standalone
// quantiser does -- the fp32 butterflies h = 1, 2, ..., d/2 (pairs (k, k + h) ->
// (a + b, a - b)), one multiply by fl32(1/sqrt d), the block max, the shared exponent
// and the rounding conversion -- so the codes are bit-identical to mxattn_quantize's.
// Butterflies 1..16 run inside each block, 32 pairs the lanes 32 apart (blocks 2s and
// 2s + 1), and 64 pairs the lane's own two blocks.
template <int D>
__device__ __forceinline__ void quantise_q_blocks(const AttnArgs& a, int64_t row, int h, Rule rule,
                                                  uint32_t (&w)[D / 64][4], int (&sc)[D / 64]) {
  constexpr int S = D / 64;
  float v[S][32];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e0 = 32 * (2 * s + h);
    if (a.q_bf16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.qraw) + row * D + e0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 u = src[k];
        v[s][8 * k + 0] = bf16lo(u.x); v[s][8 * k + 1] = bf16hi(u.x);
        v[s][8 * k + 2] = bf16lo(u.y); v[s][8 * k + 3] = bf16hi(u.y);
        v[s][8 * k + 4] = bf16lo(u.z); v[s][8 * k + 5] = bf16hi(u.z);
        v[s][8 * k + 6] = bf16lo(u.w); v[s][8 * k + 7] = bf16hi(u.w);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.qraw) + row * D + e0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 u = src[k];
        v[s][4 * k + 0] = u.x; v[s][4 * k + 1] = u.y; v[s][4 * k + 2] = u.z; v[s][4 * k + 3] = u.w;
      }
    }
  }
  if (a.q_hadamard) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hh = 1; hh < 32; hh *= 2)
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if ((k & hh) == 0) {
            const float x = v[s][k], y = v[s][k + hh];
            v[s][k] = x + y;
            v[s][k + hh] = x - y;
          }
    // h = 32: the partner lane holds the other block of the pair; the lane with the
    // higher block takes partner - own
    const uint32_t sgn = h ? 0x80000000u : 0u;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const float p = __shfl_xor(v[s][k], 32);
        v[s][k] = p + __uint_as_float(__float_as_uint(v[s][k]) ^ sgn);
      }
    if constexpr (S == 2) {  // h = 64: elements k of blocks h and 2 + h
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const float x = v[0][k], y = v[1][k];
        v[0][k] = x + y;
        v[1][k] = x - y;
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int k = 0; k < 32; ++k) v[s][k] = v[s][k] * a.q_c;
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // integer max of |bits|: NaN and Inf sort above every finite value
    uint32_t mb = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) mb = max(mb, __float_as_uint(v[s][k]) & 0x7FFFFFFFu);
    w[s][0] = w[s][1] = w[s][2] = w[s][3] = 0u;
    if (mb >= 0x7F800000u) {
      sc[s] = 0xFF;  // a non-finite block: codes 0, scale NaN, as the quantiser writes it
    } else {
      sc[s] = mx_scale_byte(mb, rule);
      quant32(v[s], sc[s], w[s]);
    }
  }
}

// One workgroup = NW waves of 32 queries.
template <int D, bool PRE, bool PNQ, bool DUMP, bool PFLOOR>
__global__ __launch_bounds__(NT, 3) void k_attn(AttnArgs a, Rule prule, int qtiles, int nblocks) {
  using G = Geo<D>;
  constexpr int S = G::S;
  constexpr int NCT = G::NCT;
  // three tile stages, declared apart so the compiler can tell a DMA into one
  // stage from reads of another and keeps the DMA in flight across those reads
  __shared__ __attribute__((aligned(16))) uint8_t st0[G::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[G::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[G::STAGE];
  __shared__ __attribute__((aligned(16))) uint32_t lones[4];

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so give
  // consecutive work items (same head, neighbouring query tiles) to the same XCD
  // and its L2 sees one head's K^/V^ stream at a time.
  const int bid = blockIdx.x;
  const int per_xcd = (int)(gridDim.x / 8);
  const int item = (bid % 8) * per_xcd + bid / 8;
  if (item >= nblocks) return;
  const int64_t head = item / qtiles;
  const int qt = item % qtiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31;
  const int h = lane >> 5;
  const int nkv = (int)a.nkv;
  const Sel sel0 = byte_sel((uint32_t)h), sel1 = byte_sel((uint32_t)(2 + h));

  const uint8_t* qc = a.qc + head * a.nq * (D / 2);
  const uint8_t* qs = a.qs + head * a.nq * (D / 32);
  const int kvp = (int)a.kv_pad;
  const int arr = 4 * kvp;  // bytes of one head's pre-arranged K (or V) scales: 512 per tile
  const TileSrc src = PRE ? TileSrc{a.kc + head * a.nkv * (D / 2), a.ksa + head * arr,
                                    a.vc + head * (int64_t)D * (kvp / 2), a.vsa + head * arr,
                                    nkv * (D / 2), arr, D * (kvp / 2), arr}
                          : TileSrc{a.kc + head * a.nkv * (D / 2), a.ks + head * a.nkv * (D / 32),
                                    a.vc + head * (int64_t)D * (kvp / 2), a.vs + head * (int64_t)D * (kvp / 32),
                                    nkv * (D / 2), nkv * (D / 32), D * (kvp / 2), D * (kvp / 32)};

  // ---- three-stage ring: tile j lives in stage j % 3; its DMA is issued two tiles
  // ahead, right after the barrier that retires the reads of the stage it reuses.  The
  // first two go out before the Q prologue, whose loads and rotation then overlap them.
  const DmaOffsets<D> dof = dma_offsets<D, PRE>(a.kv_pad, wave, lane);
  tile_dma<D, PRE>(st0, dof, src, 0, wave, lane);
  tile_dma<D, PRE>(st1, dof, src, 1, wave, lane);

  // ---- Q^ fragments (B operand of S^T), kept for the whole kv loop: lane (i, h) holds
  // blocks 2s + h of query row i.  Either read from the quantised Q^, or made here
  // from the raw query rows (the fused prologue of mxattn_forward).
  const int64_t qrow = (int64_t)qt * BR + wave * 32 + i;
  const int64_t qq = qrow < a.nq ? qrow : a.nq - 1;
  v8i qf[S];
  int qsc[S];
  {
    uint32_t w[S][4];
    int sc[S];
    if (a.qraw) {
      quantise_q_blocks<D>(a, head * a.nq + qq, h, prule, w, sc);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint4 u = *reinterpret_cast<const uint4*>(qc + qq * (D / 2) + 16 * (2 * s + h));
        w[s][0] = u.x; w[s][1] = u.y; w[s][2] = u.z; w[s][3] = u.w;
        sc[s] = qs[qq * (D / 32) + 2 * s + h];
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      qf[s] = v8i{(int)w[s][0], (int)w[s][1], (int)w[s][2], (int)w[s][3], 0, 0, 0, 0};
      qsc[s] = sc[s];
    }
  }

  // ---- online-softmax state: lane (i, h) holds channels 32 ct + 8(v/4) + 4h + v%4
  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};
  float m = -INFINITY, l = 0.0f;
  const float cl = a.scale_log2;
  const int ntiles = (nkv + BC - 1) / BC;
  const int nfull = nkv / BC;  // tiles with no padded key

  if (tid < 4) lones[tid] = 0x22222222u;
  // the first tile's barrier publishes it; that barrier does not wait for LDS writes itself
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)

  // Wait for this wave's DMAs of tile j (those of tile j + 1 may stay in flight);
  // the barrier then makes every wave's DMAs of tile j visible and guarantees that
  // every wave is done with tile j - 1, whose stage the DMA of tile j + 2 refills.
  // Past the last tile the descriptors have size zero: that DMA only writes zeros
  // into the free stage, and keeps the per-tile DMA count uniform.
  int sj = 0;  // stage of tile j
  auto enter = [&](int j) -> const uint8_t* {
    if constexpr (DUMP) MX_VMCNT(0);  // the P^ dump's stores share the counter
    else MX_VMCNT(G::NDMA);
    stage_barrier();
    uint8_t* cur = sj == 0 ? st0 : (sj == 1 ? st1 : st2);
    uint8_t* nxt = sj == 0 ? st2 : (sj == 1 ? st0 : st1);
    tile_dma<D, PRE>(nxt, dof, src, j + 2, wave, lane);
    sj = sj == 2 ? 0 : sj + 1;
    return cur;
  };
  int j = 0;
  for (; j < nfull; ++j) {
    const uint8_t* cur = enter(j);
    attend_tile<D, PRE, PNQ, DUMP, PFLOOR, false>(cur, lane, sel0, sel1, BC, qf, qsc, acc, m, l, cl, a.p_log2q, a, qrow,
                                                  head, j,
                                     lones);
  }
  if (j < ntiles) {  // the ragged last tile, masked
    const uint8_t* cur = enter(j);
    attend_tile<D, PRE, PNQ, DUMP, PFLOOR, true>(cur, lane, sel0, sel1, nkv - j * BC, qf, qsc, acc, m, l, cl, a.p_log2q,
                                                 a, qrow,
                                    head, j, lones);
  }
  MX_VMCNT(0);  // no DMA may still target this workgroup's LDS when it exits
  // Keep the last tile's MFMAs out of the epilogue's divergent branch below: an MFMA
  // reads its operands across the whole wave, so under a partial exec mask (a wave
  // holding query rows past the end) it would drop the inactive lanes' channels.
  pin_all(acc, l);

  // ---- epilogue: O = O~ / l
  if (qrow < a.nq) {
    const float inv = 1.0f / l;
    const int64_t orow = head * a.nq + qrow;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int ch = 32 * ct + 8 * b + 4 * h;
        const float o0 = acc[ct][4 * b] * inv, o1 = acc[ct][4 * b + 1] * inv;
        const float o2 = acc[ct][4 * b + 2] * inv, o3 = acc[ct][4 * b + 3] * inv;
        if (a.out_bf16) {
          uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + orow * D + ch;
          const uint32_t w0 = f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
          const uint32_t w1 = f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
          *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
        } else {
          float* op = reinterpret_cast<float*>(a.o) + orow * D + ch;
          *reinterpret_cast<float4*>(op) = make_float4(o0, o1, o2, o3);
        }
      }
  }
}

template <int D, bool PRE, bool PNQ, bool DUMP>
static void launch_rule(const AttnArgs& a, Rule pr, dim3 grid, int qtiles, int nblocks, hipStream_t s) {
  if (a.p_floor)
    hipLaunchKernelGGL((k_attn<D, PRE, PNQ, DUMP, true>), grid, dim3(NT), 0, s, a, pr, qtiles, nblocks);
  else
    hipLaunchKernelGGL((k_attn<D, PRE, PNQ, DUMP, false>), grid, dim3(NT), 0, s, a, pr, qtiles, nblocks);
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int pnq, Rule pr, hipStream_t s) {
  const int qtiles = (int)((a.nq + BR - 1) / BR);
  const int64_t nb = (int64_t)qtiles * a.heads;
  if (nb > (int64_t)0x7FFFFFF0) return hipErrorInvalidValue;
  const int nblocks = (int)nb;
  const dim3 grid((unsigned)((nblocks + 7) / 8 * 8));
  const bool dump = a.pc != nullptr;
  const bool pre = a.ksa != nullptr;
  if (pre && dump) return hipErrorInvalidValue;  // the P^ dump comes with caller-layout operands only
  if (pre && pnq) launch_rule<D, true, true, false>(a, pr, grid, qtiles, nblocks, s);
  else if (pre) launch_rule<D, true, false, false>(a, pr, grid, qtiles, nblocks, s);
  else if (pnq && !dump) launch_rule<D, false, true, false>(a, pr, grid, qtiles, nblocks, s);
  else if (pnq && dump) launch_rule<D, false, true, true>(a, pr, grid, qtiles, nblocks, s);
  else if (!dump) launch_rule<D, false, false, false>(a, pr, grid, qtiles, nblocks, s);
  else launch_rule<D, false, false, true>(a, pr, grid, qtiles, nblocks, s);
  return hipGetLastError();
}

// Pre-arranged scales (the layouts described with Geo): one thread per output dword,
// K dwords first, then V.  Keys past the last one get scale byte 0.
template <int D>
__global__ void k_arrange_scales(const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vs, int64_t heads,
                                 int nkv, int kv_pad, uint32_t* __restrict__ ksa, uint32_t* __restrict__ vsa) {
  const int64_t per_head = (int64_t)kv_pad;  // dwords per head in each layout: 128 per tile
  const int64_t total = heads * per_head;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < 2 * total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const bool isv = idx >= total;
    const int64_t r = isv ? idx - total : idx;
    const int64_t head = r / per_head;
    const int q = (int)(r % per_head);
    const int j = q >> 7, lane = (q & 127) >> 1, sc = q & 1;
    const int i = lane & 31, h = lane >> 5;
    uint32_t w = 0;
    if (!isv) {
      if (sc < D / 64) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int key = BC * j + kappa(t, i);
          if (key < nkv) w |= (uint32_t)ks[(head * nkv + key) * (D / 32) + 2 * sc + h] << (8 * t);
        }
      }
      ksa[r] = w;
    } else {
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct)
        w |= (uint32_t)vs[(head * D + 32 * ct + i) * (kv_pad / 32) + 4 * j + 2 * sc + h] << (8 * ct);
      vsa[r] = w;
    }
  }
}

hipError_t launch_arrange_scales(const uint8_t* ks, const uint8_t* vs, int64_t heads, int64_t nkv, int64_t kv_pad,
                                 int d, uint8_t* ksa, uint8_t* vsa, hipStream_t s) {
  const int64_t n = 2 * heads * kv_pad;
  const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 256 * 16);
  uint32_t* ka = reinterpret_cast<uint32_t*>(ksa);
  uint32_t* va = reinterpret_cast<uint32_t*>(vsa);
  if (d == 128)
    hipLaunchKernelGGL((k_arrange_scales<128>), dim3(grid), dim3(256), 0, s, ks, vs, heads, (int)nkv, (int)kv_pad, ka,
                       va);
  else if (d == 64)
    hipLaunchKernelGGL((k_arrange_scales<64>), dim3(grid), dim3(256), 0, s, ks, vs, heads, (int)nkv, (int)kv_pad, ka,
                       va);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int d, int pnq, Rule p_rule, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, pnq, p_rule, s);
  if (d == 64) return launch_d<64>(a, pnq, p_rule, s);
  return hipErrorInvalidValue;
}

}  // namespace mxattn
