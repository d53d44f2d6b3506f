/*
 * mxattn.h -- MXFP4 attention with Universal Optimal Scaling (UOS) and
 * Pre-Normalization Quantization (PNQ), for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described in "MXAttention: Data-Free Optimal Scaling
 * and Pre-Normalization Quantization for MXFP4 Attention" (arXiv 2607.24377;
 * abstract, and the Pith review of it: Core claim, Axiom ledger, Figures 1-4).
 * The pages describe the operator only as a directly callable MXFP4 attention
 * that drops into a video-DiT attention call (10100.com explainer, closing
 * section) and whose fused kernel needs only a changed scale-selection
 * constant plus reuse of the quantised softmax tile (Pith review, "If this is
 * right").  This header is that operator as a plain C ABI.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers; the caller allocates and owns every
 *    buffer (inputs, outputs, workspace).  The library never allocates, frees
 *    or synchronises device memory.  Work is enqueued on `stream` (a
 *    hipStream_t; NULL = the null stream) and the call returns without
 *    waiting.  Every call enqueues kernels only (no memset or copy nodes), so it
 *    can be captured into a HIP graph and replayed.
 *  - Tensors are dense, row-major (last index fastest), 16-byte aligned.
 *  - Arguments are checked on the host before any HIP call.  A failed check
 *    returns a negative mxattn_status and sets a thread-local message
 *    readable with mxattn_last_error(); nothing is launched.  A launch error
 *    returns MXATTN_E_HIP.  No C++ exception crosses the ABI.
 *  - E2M1 codes are packed two per byte, the even element in the low nibble;
 *    a code is sign << 3 | magnitude index into {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *    Scales are E8M0 bytes: value 2^(byte - 127); 0xFF marks a block that held
 *    Inf or NaN (its codes are 0).
 *  - Non-finite input.  A block holding Inf or NaN is quantised to scale 0xFF
 *    (NaN, as the OCP MX format reads that byte) with codes 0, and the attention
 *    treats it as NaN values, as IEEE arithmetic on the dequantised operands would
 *    (Pith review, Appendix A opening: the conversion routine handles values the
 *    format cannot hold): such a block in a query row makes that row of O NaN; in
 *    any key of K, every row of O (every logit with that key is NaN, and so is each
 *    row's running max); in V (32 tokens of one channel), that channel of O in
 *    every row.  The P^ dump records every tile of a NaN row as scale 0xFF, codes 0.
 *    Logits are accumulated in fp32: inputs for which softmax_scale * |q^ . k^|
 *    exceeds the fp32 range (about 3.4e38; it takes elements of magnitude above
 *    roughly 1e18) give unspecified results.
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXATTN_OK = 0,
  MXATTN_E_INVALID = -1,     /* a bad argument (null pointer, bad size, misaligned pointer, bad enum) */
  MXATTN_E_UNSUPPORTED = -2, /* a valid request this build does not implement (e.g. d not in {64,128}) */
  MXATTN_E_WORKSPACE = -3,   /* workspace smaller than mxattn_forward_workspace_bytes() */
  MXATTN_E_HIP = -4          /* the HIP runtime reported an error while launching */
} mxattn_status;

typedef enum { MXATTN_F32 = 0, MXATTN_BF16 = 1 } mxattn_dtype;

/*
 * Shared-scale rule (Pith review, Figure 3 caption; Appendix G Eq. 96):
 *  UOS  : e = smallest integer with M <= 7.25 * 2^e   (scaled max in (3.625, 7.25])
 *  OCP  : e = floor(log2 M) - 2                       (scaled max in [4, 8))
 *  CEIL : e = smallest integer with M <= qmax * 2^e, qmax in (4, 8]
 *         (qmax = 6 is TFS, qmax = 7 is OAS).
 * M is the block's max |x|.  M = 0 gives e = -127; e is clamped to [-127, 127].
 * `qmax` is read only for MXATTN_RULE_CEIL.
 */
typedef enum { MXATTN_RULE_UOS = 0, MXATTN_RULE_OCP = 1, MXATTN_RULE_CEIL = 2 } mxattn_rule_kind;

typedef enum {
  MXATTN_AXIS_LAST = 0, /* blocks of 32 along the last axis (Q and K: along the head dim) */
  MXATTN_AXIS_ROWS = 1  /* blocks of 32 down the rows (V: along tokens), output transposed */
} mxattn_axis;

/* The kv tile width B_c of the attention kernel (a multiple of 32).  PNQ's
 * quantised tile depends on it (the running max decides what is quantised), so
 * a reference that wants to reproduce the kernel's P^ must use this width and
 * visit tiles in increasing kv order. */
int32_t mxattn_kv_tile(void);

/* N rounded up to a multiple of mxattn_kv_tile(): the padded token count of the
 * transposed V layout below.  Returns -1 for N < 0. */
int64_t mxattn_padded_tokens(int64_t n);

/*
 * mxattn_quantize -- block-quantise a tensor to MXFP4 (Pith review, Axiom
 * ledger axiom 1: 32-element blocks, one E8M0 power-of-two scale, E2M1 values,
 * round to nearest with saturation; 10100.com explainer).
 *
 *   x       [batch, rows, cols] of dtype `dtype` (MXATTN_F32 or MXATTN_BF16).
 *   axis    MXATTN_AXIS_LAST: cols must be a multiple of 32; with hadamard != 0
 *             cols must be 64 or 128.
 *             codes  [batch, rows, cols/2]   scales [batch, rows, cols/32]
 *           MXATTN_AXIS_ROWS: cols must be even and <= 65536, batch <= 65535;
 *             hadamard must be 0.  With
 *             P = mxattn_padded_tokens(rows):
 *             codes  [batch, cols, P/2]      scales [batch, cols, P/32]
 *             (each column's blocks run along rows; rows past `rows` are zeros,
 *             so their blocks get scale 0x00 and codes 0).  P pads to the kv tile
 *             (mxattn_kv_tile() = 128 keys), not just to the 32-element block:
 *             this layout is the attention kernel's V^T operand, which it streams
 *             one kv tile at a time as a contiguous 64-byte run per channel, and
 *             the whole-tile padding keeps every such run inside the tensor.
 *   rule_kind, qmax   the scale rule (above).
 *   hadamard  if nonzero, each row is first rotated by the orthonormal
 *             Sylvester Hadamard matrix, y = x H / sqrt(cols), computed in
 *             fp32 as the fast Walsh-Hadamard butterflies h = 1, 2, ..., cols/2
 *             (pairs (i, i+h) -> (a+b, a-b), round to nearest even, no fused
 *             multiply-add) followed by one multiply by fl32(1/sqrt(cols))
 *             (Pith review, Axiom ledger: a fixed orthogonal Hadamard rotation
 *             on Q/K, sec. 4.3).  The codes are decided on these fp32 values.
 * Rounding: nearest E2M1 value, ties to the even code, |v| > 6 saturates to 6,
 * the sign bit is kept for values that round to zero.
 * Returns MXATTN_OK or a negative status.  batch, rows >= 1 are required.
 */
int mxattn_quantize(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols,
                    int32_t axis, int32_t rule_kind, float qmax, uint32_t hadamard,
                    uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mxattn_quant_error -- the quantisation error of mxattn_quantize, for the scale-rule
 * (Qmax) sweep that the Pith review's referee report asks for (major comments: the
 * optimality of q = 7.25 is argued for a model density, per-block sweeps on real
 * tensors, P~ tiles included, are missing).  Same arguments and checks as
 * mxattn_quantize, but nothing is stored: the blocks are quantised exactly as
 * mxattn_quantize would (after the Hadamard rotation when hadamard != 0), each code
 * is dequantised, and
 *   sums[0] = sum over finite blocks of (value - dequantised value)^2,
 *   sums[1] = sum over finite blocks of value^2,
 *   sums[2] = number of blocks left out because they hold Inf or NaN,
 * where "value" is what was quantised (the rotated fp32 value with hadamard != 0).
 * sums: 3 doubles of device memory, 8-byte aligned, owned by the caller; the call
 * zeroes them on `stream` (with a kernel) before adding.  Per-block sums are fp32,
 * the totals fp64.
 */
int mxattn_quant_error(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols,
                       int32_t axis, int32_t rule_kind, float qmax, uint32_t hadamard,
                       double* sums, void* stream);

/* Bytes of workspace mxattn_forward needs: the codes of the quantised K (along d)
 * and of the transposed quantised V (along tokens), and both scale sets, which the
 * forward's quantisers write directly in the order of mxattn_arrange_scales; each
 * piece 256-byte aligned (Q is rotated and quantised inside the attention kernel and
 * never stored).  Returns 0 for invalid sizes. */
size_t mxattn_forward_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d);

/*
 * mxattn_forward -- MXFP4 attention forward, O = softmax(scale Q K^T) V, with
 * the MXAttention pipeline (Pith review, Figure 1 caption and Figure 4; abstract):
 *   1. Q and K: optional Hadamard rotation along d, then block quantisation along d
 *      (K by the quantiser into the workspace; Q by the attention kernel as it loads
 *      its query rows -- the same arithmetic, so the same codes as mxattn_quantize).
 *   2. V: block quantisation along tokens.  The scales of K^ and V^T go into the
 *      workspace directly in the order of mxattn_arrange_scales (the same bytes that
 *      mxattn_quantize followed by mxattn_arrange_scales would give, apart from the
 *      slots of keys past Nkv, which are left unwritten and whose logits are masked).
 *      With the rotation and K, V of at most 128 MiB each, K's and V's quantisation
 *      run as one kernel launch, otherwise as two; the bytes written are the same.
 *   3. FlashAttention-2 online softmax over kv tiles of mxattn_kv_tile() keys, in
 *      increasing order.  Per tile: S = scale * (Q^ K^^T) on block-scaled MFMA;
 *      m' = max(m, rowmax S); alpha = exp(m - m'); P~ = exp(S - m').
 *      pnq != 0 (PNQ): P~ is quantised once, in 32-key blocks aligned to key 0,
 *        with the same rule, and that one P^ feeds l = alpha l + rowsum(P^) and
 *        O~ = alpha O~ + P^ V^, so the weights sum to one (Proposition 1).
 *      pnq == 0 (direct placement, Figure 4(C)): l = alpha l + rowsum(P~) while
 *        O~ still uses P^.
 *      O = O~ / l.
 *   Q [B, H, Nq, d]; K, V [B, H, Nkv, d]; O [B, H, Nq, d]; all of dtype `dtype`.
 *   d must be 64 or 128; 1 <= Nq, Nkv <= 2^24; softmax_scale finite and > 0.
 *   workspace: device memory of at least mxattn_forward_workspace_bytes(...)
 *   bytes, 256-byte aligned, owned by the caller (contents are scratch).
 * Non-causal, no mask beyond the ragged kv tail.
 */
int mxattn_forward(const void* Q, const void* K, const void* V, int32_t dtype,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                   float softmax_scale, uint32_t hadamard, uint32_t pnq,
                   int32_t rule_kind, float qmax,
                   void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxattn_forward_quantized -- step 3 of mxattn_forward on caller-supplied
 * MXFP4 operands (the layouts mxattn_quantize produces):
 *   Qc [B, H, Nq, d/2],  Qs [B, H, Nq, d/32]      (AXIS_LAST)
 *   Kc [B, H, Nkv, d/2], Ks [B, H, Nkv, d/32]     (AXIS_LAST)
 *   VTc [B, H, d, P/2],  VTs [B, H, d, P/32]      (AXIS_ROWS, P = mxattn_padded_tokens(Nkv))
 *   O [B, H, Nq, d] in out_dtype.  Shape limits as for mxattn_forward.
 *   p_rule_kind / p_qmax: the scale rule for the P~ tiles.
 *   p_codes, p_scales: either both NULL, or a dump of every quantised P^ tile:
 *   p_codes [B, H, Nq, P/2] and p_scales [B, H, Nq, P/32] (keys past Nkv have
 *   code 0; their blocks follow the rule on the zero-padded tile).
 */
int mxattn_forward_quantized(const uint8_t* Qc, const uint8_t* Qs,
                             const uint8_t* Kc, const uint8_t* Ks,
                             const uint8_t* VTc, const uint8_t* VTs,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                             float softmax_scale, uint32_t pnq,
                             int32_t p_rule_kind, float p_qmax,
                             void* O, int32_t out_dtype,
                             uint8_t* p_codes, uint8_t* p_scales, void* stream);

/*
 * mxattn_arrange_scales -- the scales of quantised K^ and V^T re-ordered, per kv
 * tile of mxattn_kv_tile() keys, into the order in which the attention kernel's
 * lanes hand them to its block-scaled MFMAs (mxattn_forward does this in its own
 * workspace).  For callers that quantise K and V once and attend to them many
 * times (cached keys and values, query chunks): arrange once, then call
 * mxattn_forward_arranged, whose kernel then needs no per-tile byte gathers.
 *   Ks  [B, H, Nkv, d/32] (AXIS_LAST), VTs [B, H, d, P/32] (AXIS_ROWS),
 *   P = mxattn_padded_tokens(Nkv).
 *   Ksa, VTsa: B*H*P*4 bytes each, 16-byte aligned, owned by the caller; per head
 *   and kv tile j, 512 bytes each.  With lane = 0..63, i = lane % 32, g = lane / 32
 *   and kappa(t, r) = 64(t/2) + 32((r/4)%2) + 16(t%2) + 4(r/8) + r%4:
 *     Ksa  dword 2 lane + s, byte t (t < 4): the Ks byte of key 128 j + kappa(t, i),
 *          block 2s + g, for s < d/64 (0 for keys past Nkv, and in dwords s >= d/64);
 *     VTsa dword 2 lane + c, byte ct: the VTs byte of channel 32 ct + i, block
 *          4 j + 2c + g, for ct < d/32 (bytes ct >= d/32 are 0).
 *   d must be 64 or 128; 1 <= Nkv <= 2^24.
 */
int mxattn_arrange_scales(const uint8_t* Ks, const uint8_t* VTs, int64_t B, int64_t H, int64_t Nkv, int64_t d,
                          uint8_t* Ksa, uint8_t* VTsa, void* stream);

/*
 * mxattn_forward_arranged -- mxattn_forward_quantized without the P^ dump, on K^ and
 * V^T scales in the order mxattn_arrange_scales writes (Qc, Qs, Kc, VTc as for
 * mxattn_forward_quantized).  This is the attention kernel mxattn_forward runs
 * after its quantisation passes; the output is bitwise that of
 * mxattn_forward_quantized on the same operands.
 */
int mxattn_forward_arranged(const uint8_t* Qc, const uint8_t* Qs,
                            const uint8_t* Kc, const uint8_t* Ksa,
                            const uint8_t* VTc, const uint8_t* VTsa,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                            float softmax_scale, uint32_t pnq,
                            int32_t p_rule_kind, float p_qmax,
                            void* O, int32_t out_dtype, void* stream);

/*
 * mxattn_forward_noalloc -- mxattn_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same arguments as mxattn_forward without the workspace, the same
 * kernels and bitwise the same O; the workspace is a device array inside the library
 * of MXATTN_NOALLOC_SCRATCH_BYTES.  The call allocates nothing.  Each GPU it runs on
 * holds its own copy of the array until the process ends; the copy's address is
 * looked up once per device, on the first call made with that device current.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams, or different host threads) race, so serialise them.
 * Returns MXATTN_E_WORKSPACE, before any HIP call, when the call needs more than the
 * array holds (mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d) > the size): at
 * d = 128 that is about 136 bytes per key per head, so 40 heads of up to about
 * 49,000 keys fit (Wan2.2-480p's 32,760 do, Wan2.2-720p's 75,600 do not).
 */
#define MXATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int mxattn_forward_noalloc(const void* Q, const void* K, const void* V, int32_t dtype,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                           float softmax_scale, uint32_t hadamard, uint32_t pnq,
                           int32_t rule_kind, float qmax, void* O, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* mxattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXATTN_H */
