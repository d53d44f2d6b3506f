// MXFP4 block quantisers for gfx950 (HBM-bound streaming kernels).
//
//  k_quant_hadamard : fused Hadamard-d rotation + block quantisation along the
//                     last axis (Q and K; the standalone quantise pass).
//  k_quant_last     : block quantisation along the last axis, no rotation.
//  k_quant_rows     : block quantisation down the rows (V along tokens), written
//                     transposed so each channel's kv codes are contiguous.
//  k_quant_kv       : the forward's K (rotation + quantisation) and V (token axis)
//                     in one launch, for K and V small enough that a launch's ramp
//                     is a visible share of the step.
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

// Quantisation error of a lane's blocks, for the Qmax-sweep diagnostic (no codes are
// stored in that mode): the sum of squared differences between the values that were
// quantised and their dequantised codes, the sum of squared values, and the number of
// blocks left out as non-finite.  Per-block sums are fp32, the running sums fp64.
struct ErrAcc {
  double e2 = 0.0, r2 = 0.0, nf = 0.0;
  __device__ __forceinline__ void add(const float* v, const uint32_t (&q)[4], int eb) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const float s = e8m0_scale(eb);
    float se = 0.0f, sr = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v2f d[4];
      d[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], s, 0);
      d[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], s, 1);
      d[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], s, 2);
      d[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], s, 3);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float a0 = v[8 * w + 2 * b], a1 = v[8 * w + 2 * b + 1];
        const float d0 = a0 - d[b].x, d1 = a1 - d[b].y;
        se += d0 * d0 + d1 * d1;
        sr += a0 * a0 + a1 * a1;
      }
    }
    e2 += se;
    r2 += sr;
  }
  // sum over the wave, then one atomic add per wave into out[0..2]
  __device__ __forceinline__ void flush(double* out) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      e2 += __shfl_xor(e2, m);
      r2 += __shfl_xor(r2, m);
      nf += __shfl_xor(nf, m);
    }
    if ((threadIdx.x & 63) == 0) {
      atomicAdd(out + 0, e2);
      atomicAdd(out + 1, r2);
      atomicAdd(out + 2, nf);
    }
  }
};


// ---------------------------------------------------------------------------
// Fused Hadamard + quantise.  D in {64, 128}; EB = bytes per input element (2 = bf16, 4 = fp32).
// One row is held by LPR = D/64 lanes, 64 elements each, so a wave handles a chunk
// of RW = 64/LPR rows at a time.  Waves work independently and persistently: wave w
// of W takes chunks w, w + W, w + 2W, ...  Each chunk is brought into the wave's own
// LDS buffer by global->LDS DMA; as soon as the lanes have read it into registers the
// DMA of the wave's next chunk is issued, so it lands while this chunk is rotated,
// quantised and stored.  In LDS, 16-byte unit q of row r sits at q ^ swz(r), which
// makes the per-lane row reads bank-conflict free.
// Butterflies h = 1..32 run inside the lane; for D = 128 the h = 64 stage pairs
// the two lanes of a row through a DPP quad permute (lanes 2r, 2r+1).
template <int D, int EB>
struct HadGeo {
  static constexpr int LPR = D / 64;          // lanes per row
  static constexpr int RW = 64 / LPR;         // rows per wave chunk
  static constexpr int RB = D * EB;           // bytes per row
  static constexpr int CH = RB / 16;          // 16-byte units per row
  static constexpr int CB = RW * RB;          // bytes per chunk (8 or 16 KB)
  static constexpr int NDMA = CB / 1024;      // 1 KB DMAs per chunk
  static constexpr int NW = 4;                // waves per workgroup
  // swizzle of row r: the 16 (or 8) lanes of one LDS read cycle hit distinct units
  __device__ static int swz(int r) {
    if constexpr (D == 128 && EB == 2) return r & 7;         // 16 units/row, lanes read 8 each
    else if constexpr (D == 64 && EB == 2) return (r >> 1) & 7;  // 8 units/row, 2 rows per 256 B
    else return r & 15;                                        // fp32: 32 or 16 units/row
  }
};

// ARR: scales go straight into the attention kernel's operand order (arr_keys rows per
// head, 4 arr_pad bytes per head) instead of [nrows, D/32].
// The body runs as workgroup `bid` of `nblk` with `lds` (NW * CB bytes) as its buffers,
// so that the forward can launch it together with the token-axis quantiser.
template <int D, int EB, bool ERR, bool ARR>
__device__ __forceinline__ void quant_hadamard_body(uint8_t* lds, int bid, int nblk, const uint8_t* __restrict__ x,
                                                    int64_t nrows, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, Rule rule, float c,
                                                    int64_t nchunks, double* err, int64_t arr_keys,
                                                    int64_t arr_pad) {
  using G = HadGeo<D, EB>;
  constexpr int LPR = G::LPR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* buf = lds + wave * G::CB;
  const int64_t W = (int64_t)nblk * G::NW;
  int64_t chunk = (int64_t)bid * G::NW + wave;
  const int64_t total = nrows * G::RB;

  // per-lane DMA source offsets within a chunk (the same for every chunk)
  uint32_t doff[G::NDMA];
#pragma unroll
  for (int u = 0; u < G::NDMA; ++u) {
    const int slot = 64 * u + lane;  // 16-byte unit of the LDS chunk
    const int r = slot / G::CH, pos = slot % G::CH;
    doff[u] = (uint32_t)(r * G::RB + 16 * (pos ^ G::swz(r)));
  }
  auto issue = [&](int64_t ch) {
    const int64_t left = total - ch * G::CB;
    const int n = left <= 0 ? 0 : (left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(x + ch * G::CB), (short)0, n, 0x00020000);
    // the lane offsets are checked against the descriptor's size: rows past the end
    // read as zero without a memory access.  The input is read once: non-temporal.
#pragma unroll
    for (int u = 0; u < G::NDMA; ++u)
      dma16_stream(rs, buf + 1024 * u, doff[u]);
  };

  const int lr = lane / LPR;    // row within the chunk
  const int half = lane % LPR;  // which 64 elements of the row
  // The stores of a chunk are issued one iteration late, after the next chunk has
  // been read from LDS: the wait for the DMA that filled the buffer, before those reads,
  // then never waits on stores issued just before it.
  uint32_t q[2][4];
  uint32_t sb2 = 0;
  int64_t prow = -1;  // row whose results q / sb2 hold (-1: none)
  ErrAcc acc;
  auto store = [&]() {
    if (!ERR && prow >= 0 && prow < nrows) {
      uint8_t* crow = codes + prow * (D / 2) + half * 32;
      *reinterpret_cast<uint4*>(crow) = make_uint4(q[0][0], q[0][1], q[0][2], q[0][3]);
      *reinterpret_cast<uint4*>(crow + 16) = make_uint4(q[1][0], q[1][1], q[1][2], q[1][3]);
      if constexpr (ARR) {
        int64_t head, key;
        split_row(prow, arr_keys, nrows, head, key);
        uint8_t* hs = scales + head * (4 * arr_pad);
        hs[arranged_k_offset(key, 2 * half)] = (uint8_t)sb2;
        hs[arranged_k_offset(key, 2 * half + 1)] = (uint8_t)(sb2 >> 8);
      } else {
        *reinterpret_cast<uint16_t*>(scales + prow * (D / 32) + half * 2) = (uint16_t)sb2;
      }
    }
  };
  if (chunk < nchunks) issue(chunk);
  for (; chunk < nchunks; chunk += W) {
    // wait until this chunk's DMA (the wave's newest vector-memory operation) has landed
    // in LDS before reading it; the stores issued before it went out an iteration ago
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    float v[64];
    {
      const uint8_t* p = buf + lr * G::RB;
      if constexpr (EB == 2) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint4 w = *reinterpret_cast<const uint4*>(p + 16 * ((8 * half + k) ^ G::swz(lr)));
          v[8 * k + 0] = bf16lo(w.x); v[8 * k + 1] = bf16hi(w.x);
          v[8 * k + 2] = bf16lo(w.y); v[8 * k + 3] = bf16hi(w.y);
          v[8 * k + 4] = bf16lo(w.z); v[8 * k + 5] = bf16hi(w.z);
          v[8 * k + 6] = bf16lo(w.w); v[8 * k + 7] = bf16hi(w.w);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float4 w = *reinterpret_cast<const float4*>(p + 16 * ((16 * half + k) ^ G::swz(lr)));
          v[4 * k + 0] = w.x; v[4 * k + 1] = w.y; v[4 * k + 2] = w.z; v[4 * k + 3] = w.w;
        }
      }
    }
    // every lane's reads of the buffer have returned: refill it with the next chunk
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    store();
    if (chunk + W < nchunks) issue(chunk + W);

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
      // a-lane: own + partner = a + b;  b-lane: partner + (-own) = a - b.  The quad
      // permute never leaves its quad, so every lane reads a partner and the move
      // folds into the add as a DPP operand.
      const uint32_t sgn = (uint32_t)half << 31;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float p = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[i]), 0xB1, 0xF, 0xF, true));
        v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ sgn);
      }
    }

    sb2 = 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float* blk = v + 32 * b;
      const uint32_t mh = absmax32_bits(blk);
#pragma unroll
      for (int i = 0; i < 32; ++i) blk[i] = blk[i] * c;
      q[b][0] = q[b][1] = q[b][2] = q[b][3] = 0u;
      uint32_t sbyte = 0xFF;
      if (mh < 0x7F800000u) {
        // max |fl(v c)| = fl(max|v| c), since rounding is monotone
        const uint32_t mb = __float_as_uint(__uint_as_float(mh) * c);
        const int eb = mx_scale_byte(mb, rule);
        quant32(blk, eb, q[b]);
        sbyte = (uint32_t)eb;
        if (ERR && chunk * G::RW + lr < nrows) acc.add(blk, q[b], eb);
      } else if (ERR && chunk * G::RW + lr < nrows) {
        acc.nf += 1.0;
      }
      sb2 |= sbyte << (8 * b);
    }
    prow = chunk * G::RW + lr;
  }
  store();
  if constexpr (ERR) acc.flush(err);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) before the wave's LDS is released
}

template <int D, int EB, bool ERR, bool ARR>
__global__ __launch_bounds__(256) void k_quant_hadamard(const uint8_t* __restrict__ x, int64_t nrows,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, Rule rule,
                                                        float c, int64_t nchunks, double* err, int64_t arr_keys,
                                                        int64_t arr_pad) {
  using G = HadGeo<D, EB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::NW * G::CB];
  quant_hadamard_body<D, EB, ERR, ARR>(lds, (int)blockIdx.x, (int)gridDim.x, x, nrows, codes, scales, rule, c,
                                       nchunks, err, arr_keys, arr_pad);
}

// ---------------------------------------------------------------------------
// Plain quantise along the last axis: one thread per 32-element block.
// ARR: scales in the attention kernel's operand order, blocks_per_row blocks per row and
// arr_keys rows per head (4 arr_pad bytes per head).
template <int EB, bool ERR, bool ARR>
__global__ __launch_bounds__(256) void k_quant_last(const uint8_t* __restrict__ x, int64_t nblocks,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, Rule rule, double* err,
                                                    int blocks_per_row, int64_t arr_keys, int64_t arr_pad) {
  const int64_t blk0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (!ERR && blk0 >= nblocks) return;
  const bool valid = blk0 < nblocks;
  const int64_t blk = valid ? blk0 : nblocks - 1;
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
  const uint32_t mb = absmax32_bits(v);
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  uint8_t sb;
  ErrAcc acc;
  if (mb >= 0x7F800000u) {
    sb = 0xFF;
    if (ERR && valid) acc.nf = 1.0;
  } else {
    const int eb = mx_scale_byte(mb, rule);
    quant32(v, eb, q);
    sb = (uint8_t)eb;
    if (ERR && valid) acc.add(v, q, eb);
  }
  if constexpr (ERR) {
    acc.flush(err);
  } else {
    *reinterpret_cast<uint4*>(codes + blk * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    if constexpr (ARR) {
      const int64_t row = blk / blocks_per_row;
      int64_t head, key;
      split_row(row, arr_keys, nblocks / blocks_per_row, head, key);
      scales[head * (4 * arr_pad) + arranged_k_offset(key, (int)(blk - row * blocks_per_row))] = sb;
    } else {
      scales[blk] = sb;
    }
  }
}

// ---------------------------------------------------------------------------
// Quantise down the rows (tokens) and write transposed:
//   x [batch, rows, cols] -> codes [batch, cols, P/2], scales [batch, cols, P/32].
// A 256-thread block owns a tile of 256 tokens x 64 columns.  The tile is brought
// into LDS by global->LDS DMA (16-byte units; tokens past `rows` read as zero through
// the buffer descriptor's size), with unit q of token r stored at q ^ ((r / 32) % 8)
// so that the column reads below spread over all banks.  Thread t then quantises
// columns 2p, 2p + 1 (p = t / 8) over the 32 tokens of block t % 8: the eight lanes
// of a column pair write the column's 128 code bytes of the tile contiguously.
// Tiles are numbered token tile fastest, then column tile, then batch item, and dealt
// to the eight XCDs in contiguous ranges (workgroups go to the XCDs round-robin): the
// tiles that complete each other's partial 128-byte lines of codes and scales (a
// channel's row is not a multiple of 128 bytes) then write through the same L2.

// ARR: scales in the attention kernel's operand order (one head per batch item, 4 P bytes
// per head) instead of [batch, cols, P/32].
// The body runs as workgroup `bid` of `nblk` (a multiple of 8, with bid on the XCD that
// hardware block bid would be dealt to) with `tile` (RowsGeo<EB>::LDS bytes) as its LDS.
template <int EB>
struct RowsGeo {
  static constexpr int TT = 256;                   // tokens per tile
  static constexpr int TC = 64;                    // columns per tile
  static constexpr int RB = TC * EB;               // bytes of one tile row: 128 (bf16) or 256 (fp32)
  static constexpr int CH = RB / 16;               // 16-byte units per tile row
  static constexpr int NDMA = TT * RB / 1024 / 4;  // 1 KB DMAs per wave
  static constexpr int LDS = TT * RB;
};

template <int EB, bool ERR, bool ARR>
__device__ __forceinline__ void quant_rows_body(uint8_t* tile, int bid, int nblk, const uint8_t* __restrict__ x,
                                                int64_t rows, int64_t cols, int64_t P, int64_t batch,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, Rule rule,
                                                double* err) {
  using RG = RowsGeo<EB>;
  constexpr int TT = RG::TT, TC = RG::TC, RB = RG::RB, CH = RG::CH, NDMA = RG::NDMA;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nx = (P + TT - 1) / TT, ny = (cols + TC - 1) / TC;
  const int64_t per_xcd = (int64_t)(nblk / 8);
  const int64_t item = (int64_t)(bid % 8) * per_xcd + bid / 8;
  if (item >= nx * ny * batch) return;
  const int64_t t0 = (item % nx) * TT;
  const int64_t c0 = ((item / nx) % ny) * TC;
  const int64_t b = item / (nx * ny);
  {
    // descriptor over this batch item from token t0, column c0 to its end
    const int64_t left = ((rows - t0) * cols - c0) * EB;
    const int n = left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(x + ((b * rows + t0) * cols + c0) * EB), (short)0, n, 0x00020000);
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const int slot = 64 * (NDMA * wave + u) + lane;  // 16-byte unit of the LDS tile
      const int r = slot / CH, pos = slot % CH;
      const int q = pos ^ (r >> 5);  // the global unit stored at `pos`
      dma16_stream(rs, tile + 1024 * (NDMA * wave + u), (uint32_t)(r * cols * EB + 16 * q));
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMAs have landed
  __syncthreads();

  const int p = tid >> 3, blk = tid & 7;
  const int sw = blk;  // (r / 32) % 8 for every token of this block
  float va[32], vb[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int r = 32 * blk + k;
    if constexpr (EB == 2) {
      // columns 2p, 2p+1: bytes 4p .. 4p+3 of the row, unit p / 4
      const uint32_t w =
          *reinterpret_cast<const uint32_t*>(tile + r * RB + 16 * ((p >> 2) ^ sw) + 4 * (p & 3));
      va[k] = bf16lo(w);
      vb[k] = bf16hi(w);
    } else {
      // bytes 8p .. 8p+7 of the row, unit p / 2
      const uint2 w = *reinterpret_cast<const uint2*>(tile + r * RB + 16 * ((p >> 1) ^ sw) + 8 * (p & 1));
      va[k] = __uint_as_float(w.x);
      vb[k] = __uint_as_float(w.y);
    }
  }
  const int64_t col = c0 + 2 * p;
  const int64_t kv0 = t0 + 32 * blk;
  if (!ERR && kv0 >= P) return;
  ErrAcc acc;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* v = s ? vb : va;
    if (kv0 >= P || col + s >= cols) break;
    const uint32_t mb = absmax32_bits(v);
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    uint8_t sb;
    if (mb >= 0x7F800000u) {
      sb = 0xFF;
      if (ERR) acc.nf += 1.0;
    } else {
      const int eb = mx_scale_byte(mb, rule);
      quant32(v, eb, q);
      sb = (uint8_t)eb;
      if (ERR) acc.add(v, q, eb);
    }
    if constexpr (!ERR) {
      const int64_t crow = b * cols + col + s;
      *reinterpret_cast<uint4*>(codes + crow * (P / 2) + kv0 / 2) = make_uint4(q[0], q[1], q[2], q[3]);
      if constexpr (ARR) scales[b * (4 * P) + arranged_v_offset((int)(col + s), kv0 / 32)] = sb;
      else scales[crow * (P / 32) + kv0 / 32] = sb;
    }
  }
  if constexpr (ERR) acc.flush(err);
}

template <int EB, bool ERR, bool ARR>
__global__ __launch_bounds__(256) void k_quant_rows(const uint8_t* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t P, int64_t batch,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, Rule rule, double* err) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[RowsGeo<EB>::LDS];
  quant_rows_body<EB, ERR, ARR>(tile, (int)blockIdx.x, (int)gridDim.x, x, rows, cols, P, batch, codes, scales, rule,
                                err);
}

// The forward's K and V quantisation in one launch: workgroups [0, nk) run the Hadamard
// quantiser over K (scales in the attention kernel's operand order), the rest the
// token-axis quantiser over V.  nk is a multiple of 8, so the V workgroups keep the
// XCD dealing their numbering assumes.  The two bodies use LDS buffers of one size.
template <int D, int EB>
__global__ __launch_bounds__(256) void k_quant_kv(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                  int64_t heads, int64_t nkv, int64_t P, uint8_t* __restrict__ kc,
                                                  uint8_t* __restrict__ ksa, uint8_t* __restrict__ vc,
                                                  uint8_t* __restrict__ vsa, Rule rule, float c, int64_t nchunks,
                                                  int nk) {
  using G = HadGeo<D, EB>;
  static_assert(G::NW * G::CB == RowsGeo<EB>::LDS, "one LDS size for both quantisers");
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::NW * G::CB];
  const int bid = (int)blockIdx.x;
  if (bid < nk)
    quant_hadamard_body<D, EB, false, true>(lds, bid, nk, k, heads * nkv, kc, ksa, rule, c, nchunks, nullptr, nkv,
                                            P);
  else
    quant_rows_body<EB, false, true>(lds, bid - nk, (int)gridDim.x - nk, v, nkv, D, P, heads, vc, vsa, rule,
                                     nullptr);
}

__global__ void k_zero_f64(double* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

// ---------------------------------------------------------------------------
// Launchers.  With err == nullptr the kernels store codes and scales; otherwise they
// store nothing and add the quantisation error sums to err[0..2] (the Qmax sweep).
template <int D, int EB, bool ERR>
static void launch_h(unsigned grid, const uint8_t* x, int64_t nrows, uint8_t* codes, uint8_t* scales, Rule rule,
                     float c, int64_t nchunks, double* err, int64_t arr_keys, int64_t arr_pad, hipStream_t s) {
  if (!ERR && arr_keys > 0)
    hipLaunchKernelGGL((k_quant_hadamard<D, EB, false, true>), dim3(grid), dim3(256), 0, s, x, nrows, codes, scales,
                       rule, c, nchunks, err, arr_keys, arr_pad);
  else
    hipLaunchKernelGGL((k_quant_hadamard<D, EB, ERR, false>), dim3(grid), dim3(256), 0, s, x, nrows, codes, scales,
                       rule, c, nchunks, err, arr_keys, arr_pad);
}

hipError_t launch_quant_hadamard(const void* x, int eb, int d, int64_t nrows, uint8_t* codes,
                                 uint8_t* scales, Rule rule, float c, double* err, hipStream_t s, int64_t arr_keys,
                                 int64_t arr_pad) {
  const int rows_per_chunk = 64 / (d / 64);
  const int64_t nchunks = (nrows + rows_per_chunk - 1) / rows_per_chunk;
  // persistent waves: as many 4-wave workgroups as fit on the 256 CUs at once (three
  // per CU for bf16 input, two for fp32, by registers and LDS), each looping over chunks
  int64_t grid = (nchunks + 3) / 4;
  const int64_t resident = 256 * (eb == 2 ? 3 : 2);
  if (grid > resident) grid = resident;
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  const unsigned g = (unsigned)grid;
  const bool e = err != nullptr;
  const int64_t ak = arr_keys, ap = arr_pad;
  if (d == 128 && eb == 2) e ? launch_h<128, 2, true>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s)
                             : launch_h<128, 2, false>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s);
  else if (d == 128 && eb == 4) e ? launch_h<128, 4, true>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s)
                                  : launch_h<128, 4, false>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s);
  else if (d == 64 && eb == 2) e ? launch_h<64, 2, true>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s)
                                 : launch_h<64, 2, false>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s);
  else if (d == 64 && eb == 4) e ? launch_h<64, 4, true>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s)
                                 : launch_h<64, 4, false>(g, xp, nrows, codes, scales, rule, c, nchunks, err, ak, ap, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_kv(const void* k, const void* v, int eb, int d, int64_t heads, int64_t nkv, int64_t P,
                          uint8_t* kc, uint8_t* ksa, uint8_t* vc, uint8_t* vsa, Rule rule, float c, hipStream_t s) {
  const int rows_per_chunk = 64 / (d / 64);
  const int64_t nchunks = (heads * nkv + rows_per_chunk - 1) / rows_per_chunk;
  int64_t nk = (nchunks + 3) / 4;  // persistent K workgroups, as launch_quant_hadamard sizes them
  const int64_t resident = 256 * (eb == 2 ? 3 : 2);
  if (nk > resident) nk = resident;
  nk = (nk + 7) / 8 * 8;  // the extra workgroups find no chunk and return
  const int64_t tiles = (P + 255) / 256 * ((d + 63) / 64) * heads;
  const int64_t nv = (tiles + 7) / 8 * 8;
  if (nk + nv > (int64_t)0x7FFFFFF0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nk + nv)), block(256);
  const uint8_t* kp = static_cast<const uint8_t*>(k);
  const uint8_t* vp = static_cast<const uint8_t*>(v);
#define MX_KV(D_, EB_) \
  hipLaunchKernelGGL((k_quant_kv<D_, EB_>), grid, block, 0, s, kp, vp, heads, nkv, P, kc, ksa, vc, vsa, rule, c, \
                     nchunks, (int)nk)
  if (d == 128 && eb == 2) MX_KV(128, 2);
  else if (d == 128 && eb == 4) MX_KV(128, 4);
  else if (d == 64 && eb == 2) MX_KV(64, 2);
  else if (d == 64 && eb == 4) MX_KV(64, 4);
  else return hipErrorInvalidValue;
#undef MX_KV
  return hipGetLastError();
}

hipError_t launch_zero_f64(double* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_f64, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_quant_last(const void* x, int eb, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                             Rule rule, double* err, hipStream_t s, int blocks_per_row, int64_t arr_keys,
                             int64_t arr_pad) {
  const int64_t grid = (nblocks + 255) / 256;
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  const dim3 g((unsigned)grid), b(256);
  const bool arr = !err && arr_keys > 0;
  if (arr && (blocks_per_row < 1 || nblocks % blocks_per_row)) return hipErrorInvalidValue;
  const int bpr = blocks_per_row;
  if (eb == 2 && err)
    hipLaunchKernelGGL((k_quant_last<2, true, false>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  else if (eb == 2 && arr)
    hipLaunchKernelGGL((k_quant_last<2, false, true>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  else if (eb == 2)
    hipLaunchKernelGGL((k_quant_last<2, false, false>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  else if (err)
    hipLaunchKernelGGL((k_quant_last<4, true, false>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  else if (arr)
    hipLaunchKernelGGL((k_quant_last<4, false, true>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  else
    hipLaunchKernelGGL((k_quant_last<4, false, false>), g, b, 0, s, xp, nblocks, codes, scales, rule, err, bpr,
                       arr_keys, arr_pad);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int eb, int64_t batch, int64_t rows, int64_t cols,
                             int64_t P, uint8_t* codes, uint8_t* scales, Rule rule, double* err, hipStream_t s,
                             bool arranged) {
  const int64_t tiles = (P + 255) / 256 * ((cols + 63) / 64) * batch;
  if (tiles > (int64_t)0x7FFFFFF0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  const bool arr = arranged && !err;
#define MX_ROWS(EB_, ERR_, ARR_)                                                                                 \
  hipLaunchKernelGGL((k_quant_rows<EB_, ERR_, ARR_>), grid, dim3(256), 0, s, xp, rows, cols, P, batch, codes, scales, \
                     rule, err)
  if (eb == 2 && err) MX_ROWS(2, true, false);
  else if (eb == 2 && arr) MX_ROWS(2, false, true);
  else if (eb == 2) MX_ROWS(2, false, false);
  else if (err) MX_ROWS(4, true, false);
  else if (arr) MX_ROWS(4, false, true);
  else MX_ROWS(4, false, false);
#undef MX_ROWS
  return hipGetLastError();
}

}  // namespace mxattn
