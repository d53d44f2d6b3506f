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
// barriers they drift out of phase, so one wave's softmax (VALU) overlaps the
// other's MFMAs.
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup

template <int D>
struct Lds {
  static constexpr int KC = BC * D / 2;         // K codes, row = key (D/2 bytes), 16-byte units swizzled
  static constexpr int KS = 512;                // K scales [g][r/4][r%4][t]
  static constexpr int VC = D * 64;             // V^T codes, row = channel (64 bytes), units swizzled
  static constexpr int VS = 512;                // V scales [g][r][ct]
  static constexpr int STAGE = KC + KS + VC + VS;
};

// LDS swizzles.  A K^ or V^T row is 64 bytes (4 units of 16 bytes; K^ rows are
// 32 bytes at D = 64).  A fragment read has 16 lanes reading 16 rows at one unit
// each; XOR-ing the unit index with these row bits makes every group of 8 lanes
// hit 8 distinct 16-byte units of a 128-byte line, and every group of 16 lanes 16
// distinct units of a 256-byte line, so the reads are conflict free whether the
// LDS serves 8 or 16 lanes of a 128-bit read per cycle.
template <int D>
__device__ __forceinline__ int k_swz(int key) {
  if constexpr (D == 128) return (((key >> 1) ^ (key >> 6)) & 1) | (((key >> 5) & 1) << 1);
  else return (key >> 5) & 1;
}
__device__ __forceinline__ int v_swz(int ch) { return (((ch >> 1) ^ (ch >> 3)) & 1) | (((ch >> 2) & 1) << 1); }

// One kv tile in flight from HBM to LDS, held in registers between the two halves
// of a loop iteration.  The loads use buffer descriptors rebuilt per tile on the
// scalar unit (base advanced to the tile, size = bytes left), with per-thread
// offsets that do not change across tiles; reads past the last key return zero.
template <int D>
struct Prefetch {
  static constexpr int KCHUNKS = BC * D / 32;  // 16-byte chunks of K codes per tile
  static constexpr int VCHUNKS = D * 4;        // 16-byte chunks of V^T codes per tile
  static constexpr int KN = (KCHUNKS + NT - 1) / NT;
  static constexpr int VN = (VCHUNKS + NT - 1) / NT;
  u32x4 k[KN];
  u32x4 v[VN];
  uint32_t sc;  // threads [0,128): the key's D/32 scale bytes; [128,128+D): the channel's 4 scale bytes
};

// Per-thread byte offsets of the tile loads (tile independent).
template <int D>
struct LoadOffsets {
  uint32_t k[Prefetch<D>::KN];
  uint32_t v[Prefetch<D>::VN];
  uint32_t sc;
};

template <int D>
__device__ __forceinline__ LoadOffsets<D> load_offsets(int64_t kv_pad, int tid) {
  constexpr int KCPR = D / 32;  // 16-byte chunks per K row
  LoadOffsets<D> o;
#pragma unroll
  for (int u = 0; u < Prefetch<D>::KN; ++u) {
    const int ci = (tid + NT * u) % Prefetch<D>::KCHUNKS;
    o.k[u] = (uint32_t)((ci / KCPR) * (D / 2) + 16 * (ci % KCPR));
  }
#pragma unroll
  for (int u = 0; u < Prefetch<D>::VN; ++u) {
    const int ci = (tid + NT * u) % Prefetch<D>::VCHUNKS;
    o.v[u] = (uint32_t)((ci / 4) * (kv_pad / 2) + 16 * (ci % 4));
  }
  o.sc = tid < BC ? (uint32_t)(tid * (D / 32)) : (uint32_t)(((tid - BC) % D) * (kv_pad / 32));
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, n, 0x00020000);
}

template <int D>
__device__ __forceinline__ void tile_load(Prefetch<D>& pf, const LoadOffsets<D>& o, const uint8_t* kc,
                                          const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int nkv,
                                          int64_t kv_pad, int j, int tid) {
  const int64_t k0 = (int64_t)j * BC;  // first key of the tile
  const __amdgpu_buffer_rsrc_t rk = rsrc(kc + k0 * (D / 2), (nkv - k0) * (D / 2));
  const __amdgpu_buffer_rsrc_t rv = rsrc(vc + j * 64, (int64_t)D * kv_pad / 2 - j * 64);
#pragma unroll
  for (int u = 0; u < Prefetch<D>::KN; ++u) pf.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k[u], 0, 0);
#pragma unroll
  for (int u = 0; u < Prefetch<D>::VN; ++u) pf.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.v[u], 0, 0);
  // waves 0-1 (threads < 128) load key scales, waves 2-3 channel scales: the branch is
  // wave-uniform, so each load sees one scalar descriptor
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < BC / 64) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(ks + k0 * (D / 32), (nkv - k0) * (D / 32));
    if constexpr (D == 128)
      pf.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, o.sc, 0, 0);
    else
      pf.sc = __builtin_amdgcn_raw_buffer_load_b16(rs, o.sc, 0, 0);
  } else {
    const __amdgpu_buffer_rsrc_t rs = rsrc(vs + j * 4, (int64_t)D * kv_pad / 32 - j * 4);
    pf.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, o.sc, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void tile_store(const Prefetch<D>& pf, uint8_t* st, int tid) {
  constexpr int KCPR = D / 32;
  uint8_t* kc = st;
  uint8_t* ksc = st + Lds<D>::KC;
  uint8_t* vc = ksc + Lds<D>::KS;
  uint8_t* vsc = vc + Lds<D>::VC;
#pragma unroll
  for (int u = 0; u < Prefetch<D>::KN; ++u) {
    const int ci = tid + NT * u;
    if (ci < Prefetch<D>::KCHUNKS) {
      const int kk = ci / KCPR, cc = ci % KCPR;
      *reinterpret_cast<u32x4*>(kc + kk * (D / 2) + 16 * (cc ^ k_swz<D>(kk))) = pf.k[u];
    }
  }
#pragma unroll
  for (int u = 0; u < Prefetch<D>::VN; ++u) {
    const int ci = tid + NT * u;
    if (ci < Prefetch<D>::VCHUNKS) {
      const int ch = ci / 4, cc = ci % 4;
      *reinterpret_cast<u32x4*>(vc + ch * 64 + 16 * (cc ^ v_swz(ch))) = pf.v[u];
    }
  }
  if (tid < BC) {
    const int kk = tid;
#pragma unroll
    for (int g = 0; g < D / 32; ++g)
      ksc[((g * 4 + kk / 32) * 4 + kk % 4) * 8 + (kk % 32) / 4] = (uint8_t)(pf.sc >> (8 * g));
  } else if (tid < BC + D) {
    const int ch = tid - BC;
#pragma unroll
    for (int g = 0; g < 4; ++g) vsc[(g * 16 + ch % 16) * 8 + ch / 16] = (uint8_t)(pf.sc >> (8 * g));
  }
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

// One kv tile for one wave's QG query groups.  `rem` (TAIL only) is the number of
// valid keys in the tile.  Three phases keep the K^ and V^ fragments from being
// live at the same time: S for every group, then softmax + PNQ per group, then
// the row-sum and P^ V^ products.
template <int D, int QG, bool PNQ, bool DUMP, bool TAIL>
__device__ __forceinline__ void attend_tile(const uint8_t* __restrict__ st, int r, int g, int rem,
                                            const v8i (&qf)[QG], const int (&qsc)[QG],
                                            v4f (&acc)[QG][D / 16], v4f (&accl)[QG], float (&m)[QG],
                                            float (&ldir)[QG], float cl, Rule prule, const AttnArgs& a,
                                            const int64_t (&qrow)[QG], int64_t head, int j,
                                            const uint8_t* lones) {
  constexpr int NCT = D / 16;
  const uint8_t* lkc = st;
  const uint8_t* lks = st + Lds<D>::KC;
  const uint8_t* lvc = lks + Lds<D>::KS;
  const uint8_t* lvs = lvc + Lds<D>::VC;
  const v4f z = v4f{0, 0, 0, 0};

  // ---- phase 1: S^T = K^ Q^^T.  MFMA t uses keys 32(r/4) + 4t + (r%4) as its 16
  // rows, so s[qg][t][jj] = S(query, key 32 g + 4 t + jj of this tile).
  v4f s[QG][8];
  {
    v8i kf[8];
    int ksw[2];
    const bool live = g < D / 32;
    const int key0 = 32 * (r >> 2) + (r & 3);  // the swizzle depends only on key bits 1, 5, 6
    const uint8_t* kb = lkc + key0 * (D / 2) + 16 * (g ^ k_swz<D>(key0));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (live) w = *reinterpret_cast<const u32x4*>(kb + 4 * t * (D / 2));
      kf[t] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    }
    uint2 s2 = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (live) s2 = *reinterpret_cast<const uint2*>(lks + ((g * 4 + (r >> 2)) * 4 + (r & 3)) * 8);
    ksw[0] = (int)s2.x;
    ksw[1] = (int)s2.y;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      s[qg][0] = mma<0>(kf[0], qf[qg], z, ksw[0], qsc[qg]);
      s[qg][1] = mma<1>(kf[1], qf[qg], z, ksw[0], qsc[qg]);
      s[qg][2] = mma<2>(kf[2], qf[qg], z, ksw[0], qsc[qg]);
      s[qg][3] = mma<3>(kf[3], qf[qg], z, ksw[0], qsc[qg]);
      s[qg][4] = mma<0>(kf[4], qf[qg], z, ksw[1], qsc[qg]);
      s[qg][5] = mma<1>(kf[5], qf[qg], z, ksw[1], qsc[qg]);
      s[qg][6] = mma<2>(kf[6], qf[qg], z, ksw[1], qsc[qg]);
      s[qg][7] = mma<3>(kf[7], qf[qg], z, ksw[1], qsc[qg]);
    }
  }

  // ---- phase 2: online softmax and PNQ quantisation of P~, per query group
  v8i pf8[QG];
  int psc[QG];
  float alpha[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    if constexpr (TAIL) {
      const int lim = rem - 32 * g;  // keys of this lane's block that exist
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (4 * t + jj >= lim) s[qg][t][jj] = -INFINITY;
    }
    // block max, row max (4 lanes), running max
    const float bm = max32(s[qg]);
    const float mnew = fmaxf(m[qg], xmax4(bm));
    alpha[qg] = __builtin_amdgcn_exp2f((m[qg] - mnew) * cl);
    m[qg] = mnew;
    const float mc = mnew * cl;
    // P~ = exp(S - m'); its block max is exp(bm - m'), exactly 1 where bm = m'
    float p[32];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        p[4 * t + jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][t][jj], cl, -mc));
    const float pm = __builtin_amdgcn_exp2f((bm - mnew) * cl);
    // PNQ: quantise P~ once, in this lane's aligned 32-key block
    const int e = mx_exponent(__float_as_uint(pm), prule);
    uint32_t pc[4];
    quant32(p, e, pc);
    pf8[qg] = v8i{(int)pc[0], (int)pc[1], (int)pc[2], (int)pc[3], 0, 0, 0, 0};
    psc[qg] = e + 127;
    if constexpr (!PNQ) {
      float ls = 0.0f;
#pragma unroll
      for (int k = 0; k < 32; ++k) ls += p[k];
      ldir[qg] = ldir[qg] * alpha[qg] + xsum4(ls);
    }
    if (DUMP && qrow[qg] < a.nq) {
      const int64_t prow = head * a.nq + qrow[qg];
      const int64_t key0 = (int64_t)j * BC + 32 * g;
      *reinterpret_cast<uint4*>(a.pc + prow * (a.kv_pad / 2) + key0 / 2) = make_uint4(pc[0], pc[1], pc[2], pc[3]);
      a.ps[prow * (a.kv_pad / 32) + key0 / 32] = (uint8_t)psc[qg];
    }
  }

  // ---- phase 3: rescale, row sum and O~^T += V^^T P^^T
  v8i vf[NCT];
  int vsw[2];
  {
    const uint8_t* vb = lvc + r * 64 + 16 * (g ^ v_swz(r));  // v_swz(16 ct + r) = v_swz(r)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(vb + ct * 16 * 64);
      vf[ct] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    }
    const uint2 s2 = *reinterpret_cast<const uint2*>(lvs + (g * 16 + r) * 8);
    vsw[0] = (int)s2.x;
    vsw[1] = (int)s2.y;
  }
  v8i ones;
  {
    // all-ones fp4 operand (code 0x2 = 1.0) for the PNQ row sum, read from LDS so it
    // does not occupy registers outside this phase
    const u32x4 w = *reinterpret_cast<const u32x4*>(lones);
    ones = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    // rescale the running state when any row's max moved (alpha == 1 is exact)
    if (__builtin_amdgcn_ballot_w64(alpha[qg] != 1.0f)) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[qg][ct] *= alpha[qg];
      accl[qg] *= alpha[qg];
    }
    // row sum: PNQ sums the same P^ with a ones MFMA (direct placement summed P~ above)
    if constexpr (PNQ) accl[qg] = mma<0>(ones, pf8[qg], accl[qg], 127, psc[qg]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if ((ct & 3) == 0) acc[qg][ct] = mma<0>(vf[ct], pf8[qg], acc[qg][ct], vsw[ct >> 2], psc[qg]);
      if ((ct & 3) == 1) acc[qg][ct] = mma<1>(vf[ct], pf8[qg], acc[qg][ct], vsw[ct >> 2], psc[qg]);
      if ((ct & 3) == 2) acc[qg][ct] = mma<2>(vf[ct], pf8[qg], acc[qg][ct], vsw[ct >> 2], psc[qg]);
      if ((ct & 3) == 3) acc[qg][ct] = mma<3>(vf[ct], pf8[qg], acc[qg][ct], vsw[ct >> 2], psc[qg]);
    }
  }
}

// One workgroup = NW waves; wave w owns QG groups of 16 queries.
template <int D, int QG, bool PNQ, bool DUMP>
__global__ __launch_bounds__(NT, 2) void k_attn(AttnArgs a, Rule prule, int qtiles, int nblocks) {
  constexpr int NCT = D / 16;  // 16-channel tiles of O
  constexpr int BR = 16 * QG * NW;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Lds<D>::STAGE + 16];
  uint8_t* const lones = lds + 2 * Lds<D>::STAGE;

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
  const int wave = tid >> 6;
  const int r = lane & 15;   // query within a 16-group / row within an MFMA tile
  const int g = lane >> 4;   // 32-wide k block of the MFMA operand
  const int nkv = (int)a.nkv;

  const uint8_t* qc = a.qc + head * a.nq * (D / 2);
  const uint8_t* qs = a.qs + head * a.nq * (D / 32);
  const uint8_t* kc = a.kc + head * a.nkv * (D / 2);
  const uint8_t* ks = a.ks + head * a.nkv * (D / 32);
  const uint8_t* vc = a.vc + head * (int64_t)D * (a.kv_pad / 2);
  const uint8_t* vs = a.vs + head * (int64_t)D * (a.kv_pad / 32);

  // ---- Q^ fragments (B operand of S^T), kept for the whole kv loop
  v8i qf[QG];
  int qsc[QG];
  int64_t qrow[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    int64_t q = (int64_t)qt * BR + wave * (16 * QG) + qg * 16 + r;
    qrow[qg] = q;
    const int64_t qq = q < a.nq ? q : a.nq - 1;
    uint4 w = make_uint4(0, 0, 0, 0);
    int sc = 127;
    if (g < D / 32) {
      w = *reinterpret_cast<const uint4*>(qc + qq * (D / 2) + 16 * g);
      sc = qs[qq * (D / 32) + g];
    }
    qf[qg] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
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

  const LoadOffsets<D> lo = load_offsets<D>(a.kv_pad, tid);
  Prefetch<D> pf;
  tile_load<D>(pf, lo, kc, ks, vc, vs, nkv, a.kv_pad, 0, tid);
  tile_store<D>(pf, lds, tid);
  if (tid == 0) *reinterpret_cast<uint4*>(lones) = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);
  __syncthreads();

  // One loop iteration on tile j held in LDS stage S, prefetching tile j+1 into the
  // other stage.  Full tiles only; the ragged last tile is handled after the loop,
  // so the loop body carries no masking.
  auto full_tile = [&](int j, auto stage) {
    constexpr int S = decltype(stage)::value;
    const bool more = j + 1 < ntiles;
    if (more) tile_load<D>(pf, lo, kc, ks, vc, vs, nkv, a.kv_pad, j + 1, tid);
    attend_tile<D, QG, PNQ, DUMP, false>(lds + S * Lds<D>::STAGE, r, g, BC, qf, qsc, acc, accl, m, ldir, cl,
                                         prule, a, qrow, head, j, lones);
    if (more) tile_store<D>(pf, lds + (1 - S) * Lds<D>::STAGE, tid);
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    full_tile(j, std::integral_constant<int, 0>{});
    full_tile(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nfull) {
    full_tile(j, std::integral_constant<int, 0>{});
    ++j;
  }
  if (j < ntiles) {
    attend_tile<D, QG, PNQ, DUMP, true>(lds + (j & 1) * Lds<D>::STAGE, r, g, nkv - j * BC, qf, qsc, acc, accl,
                                        m, ldir, cl, prule, a, qrow, head, j, lones);
  }

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
