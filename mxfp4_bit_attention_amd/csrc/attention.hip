// Fused MXFP4 attention forward with Pre-Normalization Quantization (gfx950).
//
// Method (Pith review of MXAttention, Figure 4 caption and Core claim; abstract;
// 10100.com explainer): FlashAttention-2 online softmax where the unnormalised
// exponential tile P~ = exp(S - m') is quantised to MXFP4 once, and that one
// quantised tile P^ feeds both the row-sum update and the P^ V update, so the
// normalised weights sum to one by construction.  With PNQ off the row sum
// uses the unquantised P~ (the direct placement of Figure 4(C)).
//
// Both products are block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4 with
// fp4 operands and E8M0 scales), computed transposed so that every lane owns
// one query and one aligned 32-key block:
//   S^T = K^ Q^^T  : A = 16 keys x 128 d (from LDS), B = Q^ (registers).
//                    The 16 key rows of MFMA t are keys 32(r/4) + 4t + (r%4),
//                    r = 0..15, so after the 8 MFMAs of a 128-key tile lane
//                    l holds S(query l%16, keys 32(l/16) .. 32(l/16)+31).
//   O^T += V^^T P^^T : A = 16 channels x 128 kv (from LDS), B = P^, which is
//                    exactly the lane's 32 quantised values plus their E8M0
//                    scale, so P^ never leaves registers.
// The row max needs two cross-lane steps (v_permlane16_swap, v_permlane32_swap);
// the PNQ row sum is one extra MFMA against an all-ones A operand, which sums
// the same P^ codes the P^ V product uses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mxattn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

// D = A * B + C with fp4 A and B, E8M0 scales chosen by byte OPA of sa / byte 0 of sb.
template <int OPA>
__device__ __forceinline__ v4f mma(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OPA, sa, 0, sb);
}

__device__ __forceinline__ float xmax4(float x) {
  // max over lanes l, l^16, l^32, l^48
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xsum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int BC = kKvTile;  // 128 keys per kv tile
// A workgroup is 4 waves (one per SIMD) and two workgroups share a CU: each SIMD
// then runs one wave of each, and since the workgroups synchronise on separate
// barriers they drift out of phase, so one wave's softmax overlaps the other's MFMAs.
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding: vmcnt low
// bits [3:0] and high bits [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define MX_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))

// One kv tile in LDS.  Every region is filled by global->LDS DMA, where lane L of a
// wave writes 16 (or 4) bytes at base + 16 L (or 4 L); the layouts below are chosen
// so that each MFMA fragment is one contiguous 1 KB read per wave.
//  K codes  [t][g][r] 16-byte units: unit (t, g, r) = d-block g of key kappa(t, r)
//  K scales [8 r + t] dwords: the D/32 scale bytes of key kappa(t, r)
//  V codes  [ct][g][r]: unit (ct, g, r) = keys 32 g .. 32 g + 31 of channel 16 ct + r
//  V scales [NCT r + ct] dwords: the 4 scale bytes (one per 32-key block) of channel 16 ct + r
template <int D>
struct Geo {
  static constexpr int NCT = D / 16;        // 16-channel tiles of O
  static constexpr int GK = D / 32;         // 32-element blocks per key row
  static constexpr int KC = BC * D / 2;
  static constexpr int KS = 4 * BC;
  static constexpr int VC = D * BC / 2;
  static constexpr int VS = 4 * D;
  static constexpr int OFF_KS = KC;
  static constexpr int OFF_VC = KC + KS;
  static constexpr int OFF_VS = KC + KS + VC;
  static constexpr int STAGE = KC + KS + VC + VS;
  static constexpr int CODE_DMA = D / 64;       // 1 KB code loads per wave per tile, for K and for V
  static constexpr int NDMA = 2 * CODE_DMA + 1;  // DMA instructions per wave per tile
  static_assert(KC == NW * CODE_DMA * 1024 && VC == NW * CODE_DMA * 1024, "code DMA split");
};

// The 16 keys of S^T MFMA t (t = 0..7): row r holds key 32(r/4) + 4t + (r%4), so the
// output lane (query, g) ends up with keys 32g .. 32g + 31 of the tile.
__device__ __forceinline__ int kappa(int t, int r) { return 32 * (r >> 2) + 4 * t + (r & 3); }

// Per-lane byte offsets of a wave's tile DMAs (the same for every tile).
template <int D>
struct DmaOffsets {
  uint32_t k[Geo<D>::CODE_DMA];
  uint32_t v[Geo<D>::CODE_DMA];
  uint32_t s;  // waves 0-1: key scales; waves 2-3: channel scales
};

template <int D>
__device__ __forceinline__ DmaOffsets<D> dma_offsets(int64_t kv_pad, int wave, int lane) {
  using G = Geo<D>;
  DmaOffsets<D> o;
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) {
    const int s = 64 * (G::CODE_DMA * wave + u) + lane;  // 16-byte unit of the K region
    const int t = s / (16 * G::GK), g = (s / 16) % G::GK, r = s % 16;
    o.k[u] = (uint32_t)(kappa(t, r) * (D / 2) + 16 * g);
  }
#pragma unroll
  for (int u = 0; u < G::CODE_DMA; ++u) {
    const int s = 64 * (G::CODE_DMA * wave + u) + lane;  // 16-byte unit of the V region
    const int ct = s / 64, g = (s / 16) % 4, r = s % 16;
    o.v[u] = (uint32_t)((16 * ct + r) * (kv_pad / 2) + 16 * g);
  }
  if (wave < 2) {
    const int p = 64 * wave + lane;  // dword 8 r + t of the K scale region
    o.s = (uint32_t)(kappa(p % 8, p / 8) * (D / 32));
  } else {
    const int p = (wave - 2) * (D / 2) + lane;  // dword NCT r + ct of the V scale region
    const int ch = 16 * (p % G::NCT) + p / G::NCT;
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
template <int D>
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
  if (wave < 2) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(src.ks + ks0, max(src.ks_bytes - ks0, 0));
    // a key's scales are one dword at D = 128, two bytes at D = 64
    if constexpr (D == 128) dma4(rs, st + G::OFF_KS + 256 * wave, o.s);
    else dma2(rs, st + G::OFF_KS + 256 * wave, o.s);
  } else if (lane < D / 2) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(src.vs + 4 * j, src.vs_bytes - 4 * j);
    dma4(rs, st + G::OFF_VS + 2 * D * (wave - 2), o.s);
  }
}

// Gather byte g of each of four dwords (x, y, z, w) into one dword, x in byte 0.
__device__ __forceinline__ uint32_t gather4(const u32x4& d, uint32_t sel_lo, uint32_t sel_hi) {
  return __builtin_amdgcn_perm(d.y, d.x, sel_lo) | __builtin_amdgcn_perm(d.w, d.z, sel_hi);
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

__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Max of the 32 values s[t][jj] with a max3 tree.
__device__ __forceinline__ float max32(const v4f (&s)[8]) {
  float u[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int a = 3 * i, b = 3 * i + 1, c = 3 * i + 2;
    u[i] = fmax3(s[a / 4][a % 4], s[b / 4][b % 4], s[c / 4][c % 4]);
  }
  u[10] = fmaxf(s[7][2], s[7][3]);
  const float w0 = fmax3(u[0], u[1], u[2]), w1 = fmax3(u[3], u[4], u[5]);
  const float w2 = fmax3(u[6], u[7], u[8]), w3 = fmaxf(u[9], u[10]);
  return fmaxf(fmax3(w0, w1, w2), w3);
}

// S^T MFMAs of one 16-query group: s[t][jj] = S(query, key 32 g + 4 t + jj of the tile).
__device__ __forceinline__ void s_mfma(v4f (&s)[8], const v8i (&kf)[8], const int (&ksw)[2], const v8i& qf,
                                       int qsc) {
  const v4f z = v4f{0, 0, 0, 0};
  s[0] = mma<0>(kf[0], qf, z, ksw[0], qsc);
  s[1] = mma<1>(kf[1], qf, z, ksw[0], qsc);
  s[2] = mma<2>(kf[2], qf, z, ksw[0], qsc);
  s[3] = mma<3>(kf[3], qf, z, ksw[0], qsc);
  s[4] = mma<0>(kf[4], qf, z, ksw[1], qsc);
  s[5] = mma<1>(kf[5], qf, z, ksw[1], qsc);
  s[6] = mma<2>(kf[6], qf, z, ksw[1], qsc);
  s[7] = mma<3>(kf[7], qf, z, ksw[1], qsc);
}

// Softmax, plain-ALU part: masks keys past the end (TAIL), updates the running max m
// from the block max and the row max over the 4 lanes of the query, and turns s into
// the exponent arguments x = (S - m') * softmax_scale * log2(e).  Returns the block
// max's argument (bm - m') * cl; alpha = exp2((m - m') cl) is the running-state factor.
template <bool TAIL>
__device__ __forceinline__ float soft_alu(v4f (&s)[8], float& m, float cl, int lim, float& alpha) {
  if constexpr (TAIL) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (4 * t + jj >= lim) s[t][jj] = -INFINITY;
  }
  const float bm = max32(s);
  const float mnew = fmaxf(m, xmax4(bm));
  alpha = __builtin_amdgcn_exp2f((m - mnew) * cl);
  m = mnew;
  const float mc = mnew * cl;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) s[t][jj] = __builtin_fmaf(s[t][jj], cl, -mc);
  return (bm - mnew) * cl;
}

// Softmax, transcendental part: P~ = exp2(x) and its PNQ quantisation, once, in the
// lane's aligned 32-key block.  The block max of P~ is exp2 of the block max's
// argument (exactly 1 where the block holds the row max).
__device__ __forceinline__ void soft_exp(const v4f (&x)[8], float xm, Rule prule, float (&p)[32], uint32_t (&pc)[4],
                                         int& psc) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) p[4 * t + jj] = __builtin_amdgcn_exp2f(x[t][jj]);
  const float pm = __builtin_amdgcn_exp2f(xm);
  const int e = mx_exponent(__float_as_uint(pm), prule);
  quant32(p, e, pc);
  psc = e + 127;
}

// O~^T += V^^T P^^T for one group, plus the PNQ row sum as a ones MFMA over the same P^.
template <int D, bool PNQ>
__device__ __forceinline__ void pv_mfma(v4f (&acc)[D / 16], v4f& accl, const v8i (&vf)[D / 16], const int (&vsw)[2],
                                        const v8i& ones, const v8i& pf8, int psc) {
  constexpr int NCT = D / 16;
  if constexpr (PNQ) accl = mma<0>(ones, pf8, accl, 127, psc);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if ((ct & 3) == 0) acc[ct] = mma<0>(vf[ct], pf8, acc[ct], vsw[ct >> 2], psc);
    if ((ct & 3) == 1) acc[ct] = mma<1>(vf[ct], pf8, acc[ct], vsw[ct >> 2], psc);
    if ((ct & 3) == 2) acc[ct] = mma<2>(vf[ct], pf8, acc[ct], vsw[ct >> 2], psc);
    if ((ct & 3) == 3) acc[ct] = mma<3>(vf[ct], pf8, acc[ct], vsw[ct >> 2], psc);
  }
}

// Make the compiler produce the eight accumulator tiles at this point of the program
// (it would otherwise sink work past the branches that follow).
__device__ __forceinline__ void pin(v4f (&x)[8]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
}

// Interleave the next N MFMAs of the scheduling region with K ALU/transcendental
// instructions each, so the exponentials and conversions of one group execute in
// the shadow of the other group's matrix products.
template <int N, int K>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, K, 0);  // K VALU / TRANS
  }
}

// One kv tile for one wave's two 16-query groups (q0, q1).  The order overlaps
// each group's transcendental softmax work with the other group's MFMAs:
//   S(q0) | ALU(q0) | S(q1) + EXP(q0) | ALU(q1) | rescale | PV(q0) + EXP(q1) | PV(q1)
// `rem` (TAIL only) is the number of valid keys in the tile.
template <int D, int QG, bool PNQ, bool DUMP, bool TAIL>
__device__ __forceinline__ void attend_tile(const uint8_t* __restrict__ st, int lane, uint32_t sel_lo,
                                            uint32_t sel_hi, int rem, const v8i (&qf)[QG], const int (&qsc)[QG],
                                            v4f (&acc)[QG][D / 16], v4f (&accl)[QG], float (&m)[QG],
                                            float (&ldir)[QG], float cl, Rule prule, const AttnArgs& a,
                                            const int64_t (&qrow)[QG], int64_t head, int j,
                                            const uint32_t* lones) {
  static_assert(QG == 2, "the tile schedule pairs two query groups");
  using G = Geo<D>;
  constexpr int NCT = G::NCT;
  const int r = lane & 15;  // query within a 16-group / row within an MFMA tile
  const int g = lane >> 4;  // 32-wide k block of the MFMA operand
  const int lim = rem - 32 * g;  // keys of this lane's block that exist (TAIL)

  // K^ fragments: MFMA t uses keys kappa(t, r) as its 16 rows
  v8i kf[8];
  int ksw[2];
  {
    const bool live = g < G::GK;  // at D = 64 lanes with g >= 2 carry zero operands
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (live) w = *reinterpret_cast<const u32x4*>(st + 256 * G::GK * t + 16 * lane);
      kf[t] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    }
    // the scales of keys kappa(0..7, r): byte g of dwords 8r .. 8r + 7
    const u32x4 s0 = *reinterpret_cast<const u32x4*>(st + G::OFF_KS + 32 * r);
    const u32x4 s1 = *reinterpret_cast<const u32x4*>(st + G::OFF_KS + 32 * r + 16);
    ksw[0] = (int)gather4(s0, sel_lo, sel_hi);
    ksw[1] = (int)gather4(s1, sel_lo, sel_hi);
  }

  v4f s0[8], s1[8];
  float alpha0, alpha1, p[32];
  int psc0, psc1;
  uint32_t pc0[4], pc1[4];

  s_mfma(s0, kf, ksw, qf[0], qsc[0]);
  const float xm0 = soft_alu<TAIL>(s0, m[0], cl, lim, alpha0);
  pin(s0);
  __builtin_amdgcn_sched_barrier(0);
  s_mfma(s1, kf, ksw, qf[1], qsc[1]);
  soft_exp(s0, xm0, prule, p, pc0, psc0);
  if constexpr (!PNQ) {
    float ls = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) ls += p[k];
    ldir[0] = ldir[0] * alpha0 + xsum4(ls);
  }
  interleave_mfma<8, 6>();
  // keep group 0's quantisation here: its only consumers come after the rescale
  // branches below, past which the compiler would otherwise sink it
  asm volatile("" : "+v"(pc0[0]), "+v"(pc0[1]), "+v"(pc0[2]), "+v"(pc0[3]), "+v"(psc0));
  __builtin_amdgcn_sched_barrier(0);
  const float xm1 = soft_alu<TAIL>(s1, m[1], cl, lim, alpha1);
  pin(s1);

  // V^ fragments (A operand of O^T): channels 16 ct + r, keys 32 g .. 32 g + 31
  v8i vf[NCT];
  int vsw[2];
  {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(st + G::OFF_VC + 1024 * ct + 16 * lane);
      vf[ct] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    }
    // the scales of channels 16 ct + r: byte g of dwords NCT r .. NCT r + NCT - 1
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(st + G::OFF_VS + 4 * NCT * r);
    vsw[0] = (int)gather4(v0, sel_lo, sel_hi);
    if constexpr (NCT > 4) {
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(st + G::OFF_VS + 4 * NCT * r + 16);
      vsw[1] = (int)gather4(v1, sel_lo, sel_hi);
    } else {
      vsw[1] = 0;
    }
  }
  v8i ones;
  {
    // all-ones fp4 operand (code 0x2 = 1.0) for the PNQ row sum, read from LDS so it
    // does not occupy registers outside this phase
    const u32x4 w = *reinterpret_cast<const u32x4*>(lones);
    ones = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  }
  // rescale the running state of a group when any of its rows' max moved (alpha == 1 is exact)
  if (__builtin_amdgcn_ballot_w64(alpha0 != 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[0][ct] *= alpha0;
    accl[0] *= alpha0;
  }
  if (__builtin_amdgcn_ballot_w64(alpha1 != 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[1][ct] *= alpha1;
    accl[1] *= alpha1;
  }
  __builtin_amdgcn_sched_barrier(0);
  pv_mfma<D, PNQ>(acc[0], accl[0], vf, vsw, ones, v8i{(int)pc0[0], (int)pc0[1], (int)pc0[2], (int)pc0[3], 0, 0, 0, 0},
                  psc0);
  soft_exp(s1, xm1, prule, p, pc1, psc1);
  if constexpr (!PNQ) {
    float ls = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) ls += p[k];
    ldir[1] = ldir[1] * alpha1 + xsum4(ls);
  }
  interleave_mfma<NCT + 1, 6>();
  __builtin_amdgcn_sched_barrier(0);
  pv_mfma<D, PNQ>(acc[1], accl[1], vf, vsw, ones, v8i{(int)pc1[0], (int)pc1[1], (int)pc1[2], (int)pc1[3], 0, 0, 0, 0},
                  psc1);

  if constexpr (DUMP) {
    const uint32_t* pcs[2] = {pc0, pc1};
    const int pscs[2] = {psc0, psc1};
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      if (qrow[qg] < a.nq) {
        const int64_t prow = head * a.nq + qrow[qg];
        const int64_t key0 = (int64_t)j * BC + 32 * g;
        *reinterpret_cast<uint4*>(a.pc + prow * (a.kv_pad / 2) + key0 / 2) =
            make_uint4(pcs[qg][0], pcs[qg][1], pcs[qg][2], pcs[qg][3]);
        a.ps[prow * (a.kv_pad / 32) + key0 / 32] = (uint8_t)pscs[qg];
      }
    }
  }
}

// Fused Q quantisation (mxattn_forward): lane (r, g) turns elements 32g .. 32g + 31 of
// query row `row` into one MXFP4 block exactly as the standalone quantiser does -- the
// fp32 butterflies h = 1, 2, ..., d/2 (pairs (i, i + h) -> (a + b, a - b)), one multiply
// by fl32(1/sqrt d), the block max, the shared exponent and the rounding conversion --
// so the codes are bit-identical to mxattn_quantize's.  Butterflies h = 1..16 run in the
// lane; h = 32 and h = 64 pair the lanes holding blocks g ^ 1 and g ^ 2 (16 and 32 lanes
// apart).  Every lane of the wave takes part in the exchanges; lanes with g >= d/32 hold
// zeros and produce code 0 with scale 127.
template <int D>
__device__ __forceinline__ void quantise_q_block(const AttnArgs& a, int64_t row, int g, Rule rule,
                                                 uint32_t (&w)[4], int& sc) {
  constexpr int GK = D / 32;
  float v[32];
  if (g < GK) {
    if (a.q_bf16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.qraw) + row * D + 32 * g);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 u = src[k];
        v[8 * k + 0] = bf16lo(u.x); v[8 * k + 1] = bf16hi(u.x);
        v[8 * k + 2] = bf16lo(u.y); v[8 * k + 3] = bf16hi(u.y);
        v[8 * k + 4] = bf16lo(u.z); v[8 * k + 5] = bf16hi(u.z);
        v[8 * k + 6] = bf16lo(u.w); v[8 * k + 7] = bf16hi(u.w);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.qraw) + row * D + 32 * g);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 u = src[k];
        v[4 * k + 0] = u.x; v[4 * k + 1] = u.y; v[4 * k + 2] = u.z; v[4 * k + 3] = u.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  if (a.q_hadamard) {
#pragma unroll
    for (int h = 1; h < 32; h *= 2) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & h) == 0) {
          const float x = v[i], y = v[i + h];
          v[i] = x + y;
          v[i + h] = x - y;
        }
      }
    }
#pragma unroll
    for (int st = 1; st < GK; st *= 2) {  // h = 32 st: the partner holds block g ^ st
      const uint32_t sgn = (uint32_t)(g & st) != 0 ? 0x80000000u : 0u;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float p = __shfl_xor(v[i], 16 * st);
        v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ sgn);  // a + b, or b-lane: a + (-b)
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] * a.q_c;
  }
  if (g >= GK) return;
  // integer max of |bits| (this file is built assuming no NaNs, so no float max here):
  // NaN and Inf sort above every finite value
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  if (mb >= 0x7F800000u) {
    sc = 0xFF;  // a non-finite block: codes 0, scale NaN, as the quantiser writes it
    return;
  }
  const int e = mx_exponent(mb, rule);
  quant32(v, e, w);
  sc = e + 127;
}

// One workgroup = NW waves; wave w owns QG groups of 16 queries.
template <int D, int QG, bool PNQ, bool DUMP>
__global__ __launch_bounds__(NT, 2) void k_attn(AttnArgs a, Rule prule, int qtiles, int nblocks) {
  using G = Geo<D>;
  constexpr int NCT = G::NCT;       // 16-channel tiles of O
  constexpr int BR = 16 * QG * NW;  // queries per workgroup
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
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nkv = (int)a.nkv;
  // v_perm selectors that pick byte g of two dwords (low and high halves of gather4)
  const uint32_t sel_lo = (uint32_t)g | ((uint32_t)(g + 4) << 8) | 0x0C0C0000u;
  const uint32_t sel_hi = 0x00000C0Cu | ((uint32_t)g << 16) | ((uint32_t)(g + 4) << 24);

  const uint8_t* qc = a.qc + head * a.nq * (D / 2);
  const uint8_t* qs = a.qs + head * a.nq * (D / 32);
  const int kvp = (int)a.kv_pad;
  const TileSrc src{a.kc + head * a.nkv * (D / 2), a.ks + head * a.nkv * (D / 32),
                    a.vc + head * (int64_t)D * (kvp / 2), a.vs + head * (int64_t)D * (kvp / 32),
                    nkv * (D / 2), nkv * (D / 32), D * (kvp / 2), D * (kvp / 32)};

  // ---- Q^ fragments (B operand of S^T), kept for the whole kv loop: lane (r, g) holds
  // block g of query row r.  Either read from the quantised Q^, or made here from the
  // raw query rows (the fused prologue of mxattn_forward), see quantise_q_block.
  v8i qf[QG];
  int qsc[QG];
  int64_t qrow[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int64_t q = (int64_t)qt * BR + wave * (16 * QG) + qg * 16 + r;
    qrow[qg] = q;
    const int64_t qq = q < a.nq ? q : a.nq - 1;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    int sc = 127;
    if (a.qraw) {
      quantise_q_block<D>(a, head * a.nq + qq, g, prule, w, sc);
    } else if (g < G::GK) {
      const uint4 u = *reinterpret_cast<const uint4*>(qc + qq * (D / 2) + 16 * g);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
      sc = qs[qq * (D / 32) + g];
    }
    qf[qg] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
    qsc[qg] = sc;
  }

  // ---- online-softmax state
  v4f acc[QG][NCT];
  v4f accl[QG];
  float m[QG], ldir[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    m[qg] = -INFINITY;
    ldir[qg] = 0.0f;
    accl[qg] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[qg][ct] = v4f{0, 0, 0, 0};
  }
  const float cl = a.scale_log2;
  const int ntiles = (nkv + BC - 1) / BC;
  const int nfull = nkv / BC;  // tiles with no padded key

  // ---- three-stage ring: tile j lives in stage j % 3; its DMA is issued two tiles
  // ahead, right after the barrier that retires the reads of the stage it reuses.
  const DmaOffsets<D> dof = dma_offsets<D>(a.kv_pad, wave, lane);
  tile_dma<D>(st0, dof, src, 0, wave, lane);
  tile_dma<D>(st1, dof, src, 1, wave, lane);
  if (tid < 4) lones[tid] = 0x22222222u;

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
    tile_dma<D>(nxt, dof, src, j + 2, wave, lane);
    sj = sj == 2 ? 0 : sj + 1;
    return cur;
  };
  // The loop is not unrolled over the three stages: the stage pointers are then
  // run-time values, and the compiler adds a wait for the DMAs of the previous tile
  // (issued a whole tile earlier) before the first read, never for the ones just issued.
  int j = 0;
  for (; j < nfull; ++j) {
    const uint8_t* cur = enter(j);
    attend_tile<D, QG, PNQ, DUMP, false>(cur, lane, sel_lo, sel_hi, BC, qf, qsc, acc, accl, m, ldir, cl, prule,
                                         a, qrow, head, j, lones);
  }
  if (j < ntiles) {  // the ragged last tile, masked
    const uint8_t* cur = enter(j);
    attend_tile<D, QG, PNQ, DUMP, true>(cur, lane, sel_lo, sel_hi, nkv - j * BC, qf, qsc, acc, accl, m, ldir, cl,
                                        prule, a, qrow, head, j, lones);
  }
  MX_VMCNT(0);  // no DMA may still target this workgroup's LDS when it exits

  // ---- epilogue: O = O~ / l ; lane holds channels 16ct + 4g + jj of its query
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    if (qrow[qg] >= a.nq) continue;
    const float l = PNQ ? accl[qg][0] : ldir[qg];
    const float inv = 1.0f / l;
    const int64_t orow = head * a.nq + qrow[qg];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ch = 16 * ct + 4 * g;
      const float o0 = acc[qg][ct][0] * inv, o1 = acc[qg][ct][1] * inv;
      const float o2 = acc[qg][ct][2] * inv, o3 = acc[qg][ct][3] * inv;
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

template <int D, int QG>
static hipError_t launch_dq(const AttnArgs& a, int pnq, Rule pr, hipStream_t s) {
  constexpr int BR = 16 * QG * NW;
  const int qtiles = (int)((a.nq + BR - 1) / BR);
  const int64_t nb = (int64_t)qtiles * a.heads;
  if (nb > (int64_t)0x7FFFFFF0) return hipErrorInvalidValue;
  const int nblocks = (int)nb;
  const unsigned grid = (unsigned)((nblocks + 7) / 8 * 8);
  const bool dump = a.pc != nullptr;
  if (pnq && !dump)
    hipLaunchKernelGGL((k_attn<D, QG, true, false>), dim3(grid), dim3(NT), 0, s, a, pr, qtiles, nblocks);
  else if (pnq && dump)
    hipLaunchKernelGGL((k_attn<D, QG, true, true>), dim3(grid), dim3(NT), 0, s, a, pr, qtiles, nblocks);
  else if (!dump)
    hipLaunchKernelGGL((k_attn<D, QG, false, false>), dim3(grid), dim3(NT), 0, s, a, pr, qtiles, nblocks);
  else
    hipLaunchKernelGGL((k_attn<D, QG, false, true>), dim3(grid), dim3(NT), 0, s, a, pr, qtiles, nblocks);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int d, int pnq, Rule p_rule, hipStream_t s) {
  if (d == 128) return launch_dq<128, 2>(a, pnq, p_rule, s);
  if (d == 64) return launch_dq<64, 2>(a, pnq, p_rule, s);
  return hipErrorInvalidValue;
}

}  // namespace mxattn
