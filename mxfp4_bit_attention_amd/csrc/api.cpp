// C ABI of libmxattn: argument checks on the host, workspace carving, and
// dispatch to the HIP kernels.  Every check runs before the first HIP call, so
// a rejected call touches no device state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"
#include "mxattn.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return MXATTN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MXATTN_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t n, int64_t m) { return (n + m - 1) / m * m; }

// Largest element count accepted for one tensor (keeps every byte offset and
// grid size far inside int64 / 31-bit grid limits).
constexpr int64_t kMaxElems = int64_t(1) << 40;
// Tokens per head (Nq, Nkv) of the attention entry points: keeps every per-head byte
// count of the kernels below 2^31.
constexpr int64_t kMaxTokens = int64_t(1) << 24;
// Largest K (and V) input, in bytes, that the forward quantises in one joint launch.
constexpr int64_t kJointQuantBytes = int64_t(128) << 20;

bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > limit / a) return false;
  *out = a * b;
  return true;
}

bool elems(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* out) {
  int64_t t;
  return mul_ok(a, b, kMaxElems, &t) && mul_ok(t, c, kMaxElems, &t) && mul_ok(t, d, kMaxElems, out);
}

int make_rule(int32_t kind, float qmax, mxattn::Rule* r, const char* who) {
  float q;
  if (kind == MXATTN_RULE_UOS) {
    q = 7.25f;
  } else if (kind == MXATTN_RULE_OCP) {
    r->q_exp = 2;             // e = E - 2 ...
    r->q_frac = 0xFFFFFFFFu;  // ... whatever the fraction
    return MXATTN_OK;
  } else if (kind == MXATTN_RULE_CEIL) {
    if (!std::isfinite(qmax) || !(qmax > 4.0f) || !(qmax <= 8.0f))
      return fail(MXATTN_E_INVALID, "%s: ceil rule needs qmax in (4, 8], got %g", who, (double)qmax);
    q = qmax;
  } else {
    return fail(MXATTN_E_INVALID, "%s: unknown rule kind %d", who, (int)kind);
  }
  uint32_t b;
  std::memcpy(&b, &q, 4);
  r->q_exp = (int)(b >> 23) - 127;
  r->q_frac = b & 0x7FFFFFu;
  return MXATTN_OK;
}

int elem_bytes(int32_t dtype) { return dtype == MXATTN_F32 ? 4 : dtype == MXATTN_BF16 ? 2 : 0; }

float inv_sqrt_f32(int d) { return (float)(1.0 / std::sqrt((double)d)); }

struct Carve {
  size_t off = 0;
  size_t take(size_t n) {
    size_t o = off;
    off = (off + n + 255) / 256 * 256;
    return o;
  }
};

struct FwdLayout {
  size_t kc, vc, ksa, vsa, total;
};

// The forward's workspace: the codes of K^ and V^T (Q is quantised inside the attention
// kernel), and their scales, which the quantisers write straight into the attention
// kernel's per-tile operand order.
bool fwd_layout(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, FwdLayout* L) {
  int64_t nq_e, nkv_e, v_e;
  const int64_t P = round_up(Nkv, mxattn::kKvTile);
  if (!elems(B, H, Nq, d, &nq_e) || !elems(B, H, Nkv, d, &nkv_e) || !elems(B, H, P, d, &v_e)) return false;
  Carve c;
  L->kc = c.take((size_t)nkv_e / 2);
  L->vc = c.take((size_t)v_e / 2);
  L->ksa = c.take((size_t)(B * H * P) * 4);
  L->vsa = c.take((size_t)(B * H * P) * 4);
  L->total = c.off;
  return true;
}

int check_attn_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float softmax_scale,
                     const char* who) {
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1)
    return fail(MXATTN_E_INVALID, "%s: B, H, Nq, Nkv must be >= 1 (got %lld, %lld, %lld, %lld)", who,
                (long long)B, (long long)H, (long long)Nq, (long long)Nkv);
  if (d != 64 && d != 128) return fail(MXATTN_E_UNSUPPORTED, "%s: d must be 64 or 128, got %lld", who, (long long)d);
  if (Nq > kMaxTokens || Nkv > kMaxTokens)
    return fail(MXATTN_E_INVALID, "%s: Nq and Nkv must be <= %lld tokens per head", who, (long long)kMaxTokens);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(MXATTN_E_INVALID, "%s: softmax_scale must be finite and > 0", who);
  int64_t t;
  if (!elems(B, H, Nq > Nkv ? Nq : Nkv, d, &t) || !elems(B, H, round_up(Nkv, mxattn::kKvTile), d, &t))
    return fail(MXATTN_E_INVALID, "%s: tensor too large", who);
  if (B * H > 65535) return fail(MXATTN_E_INVALID, "%s: B * H must be <= 65535", who);
  if (B * H * ((Nq + 127) / 128) > (int64_t)0x7FFFFF00)
    return fail(MXATTN_E_INVALID, "%s: too many query tiles for one launch", who);
  return MXATTN_OK;
}

}  // namespace

extern "C" {

int32_t mxattn_kv_tile(void) { return mxattn::kKvTile; }

int64_t mxattn_padded_tokens(int64_t n) { return n < 0 ? -1 : round_up(n, mxattn::kKvTile); }

const char* mxattn_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// Shared by mxattn_quantize (err == nullptr: store codes and scales) and
// mxattn_quant_error (err != nullptr: store nothing, sum the quantisation error).
int quantize_impl(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols, int32_t axis,
                  int32_t rule_kind, float qmax, uint32_t hadamard, uint8_t* codes, uint8_t* scales, double* err,
                  void* stream, const char* who) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(MXATTN_E_INVALID, "%s: dtype must be MXATTN_F32 or MXATTN_BF16", who);
  if (!x || (!err && (!codes || !scales))) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if (!aligned16(x) || (!err && (!aligned16(codes) || !aligned16(scales))))
    return fail(MXATTN_E_INVALID, "%s: pointers must be 16-byte aligned", who);
  if (err && (reinterpret_cast<uintptr_t>(err) & 7))
    return fail(MXATTN_E_INVALID, "%s: sums must be 8-byte aligned", who);
  if (batch < 1 || rows < 1 || cols < 1)
    return fail(MXATTN_E_INVALID, "%s: batch, rows, cols must be >= 1", who);
  int64_t n;
  if (!elems(batch, rows, cols, 1, &n)) return fail(MXATTN_E_INVALID, "%s: tensor too large", who);
  mxattn::Rule rule{};
  if (int st = make_rule(rule_kind, qmax, &rule, who)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (axis == MXATTN_AXIS_LAST) {
    if (cols % 32) return fail(MXATTN_E_INVALID, "%s: cols must be a multiple of 32 for AXIS_LAST", who);
    if (hadamard && cols != 64 && cols != 128)
      return fail(MXATTN_E_UNSUPPORTED, "%s: the Hadamard rotation supports cols 64 or 128, got %lld", who,
                  (long long)cols);
  } else if (axis == MXATTN_AXIS_ROWS) {
    if (hadamard) return fail(MXATTN_E_INVALID, "%s: AXIS_ROWS does not take a Hadamard rotation", who);
    if (cols % 2) return fail(MXATTN_E_INVALID, "%s: cols must be even for AXIS_ROWS", who);
    if (batch > 65535 || cols > 65536)
      return fail(MXATTN_E_INVALID, "%s: AXIS_ROWS needs batch <= 65535 and cols <= 65536", who);
  } else {
    return fail(MXATTN_E_INVALID, "%s: axis must be MXATTN_AXIS_LAST or MXATTN_AXIS_ROWS", who);
  }
  hipError_t e = hipSuccess;
  // a kernel rather than a memset clears the sums, so the call can be captured in a graph
  if (err) e = mxattn::launch_zero_f64(err, 3, s);
  if (e == hipSuccess) {
    if (axis == MXATTN_AXIS_LAST && hadamard)
      e = mxattn::launch_quant_hadamard(x, eb, (int)cols, batch * rows, codes, scales, rule, inv_sqrt_f32((int)cols),
                                        err, s);
    else if (axis == MXATTN_AXIS_LAST)
      e = mxattn::launch_quant_last(x, eb, n / 32, codes, scales, rule, err, s);
    else
      e = mxattn::launch_quant_rows(x, eb, batch, rows, cols, round_up(rows, mxattn::kKvTile), codes, scales, rule,
                                    err, s);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

}  // namespace

extern "C" {

int mxattn_quantize(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols,
                    int32_t axis, int32_t rule_kind, float qmax, uint32_t hadamard,
                    uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_impl(x, dtype, batch, rows, cols, axis, rule_kind, qmax, hadamard, codes, scales, nullptr, stream,
                       "mxattn_quantize");
}

int mxattn_quant_error(const void* x, int32_t dtype, int64_t batch, int64_t rows, int64_t cols, int32_t axis,
                       int32_t rule_kind, float qmax, uint32_t hadamard, double* sums, void* stream) {
  if (!sums) return fail(MXATTN_E_INVALID, "mxattn_quant_error: null pointer");
  return quantize_impl(x, dtype, batch, rows, cols, axis, rule_kind, qmax, hadamard, nullptr, nullptr, sums, stream,
                       "mxattn_quant_error");
}

size_t mxattn_forward_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d) {
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || (d != 64 && d != 128)) return 0;
  FwdLayout L;
  if (!fwd_layout(B, H, Nq, Nkv, d, &L)) return 0;
  return L.total;
}

// Raw Q for the fused quantisation in the attention kernel's prologue.
struct QuantQ {
  const void* q;
  bool bf16;
  bool hadamard;
  float c;
};

static int attention_core(const uint8_t* Qc, const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                          const uint8_t* VTc, const uint8_t* VTs, int64_t B, int64_t H, int64_t Nq,
                          int64_t Nkv, int64_t d, float softmax_scale, uint32_t pnq,
                          const mxattn::Rule& pr, void* O, int32_t out_dtype, uint8_t* pc, uint8_t* ps,
                          hipStream_t s, const char* who, const QuantQ* fused = nullptr,
                          const uint8_t* ksa = nullptr, const uint8_t* vsa = nullptr) {
  mxattn::AttnArgs a{};
  a.qc = Qc;
  a.qs = Qs;
  a.kc = Kc;
  a.ks = Ks;
  a.vc = VTc;
  a.vs = VTs;
  a.ksa = ksa;
  a.vsa = vsa;
  a.o = O;
  a.pc = pc;
  a.ps = ps;
  a.heads = B * H;
  a.nq = Nq;
  a.nkv = Nkv;
  a.kv_pad = round_up(Nkv, mxattn::kKvTile);
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  a.out_bf16 = out_dtype == MXATTN_BF16;
  // the P~ rule for the kernel's log-domain block exponent (Rule's OCP encoding has a
  // fraction threshold no fraction exceeds; CEIL(q) has q = (1 + q_frac / 2^23) 2^q_exp)
  a.p_floor = pr.q_frac > 0x7FFFFFu ? 1 : 0;
  a.p_log2q = a.p_floor ? 0.0f : (float)std::log2(std::ldexp(1.0 + pr.q_frac / 8388608.0, pr.q_exp));
  if (fused) {
    a.qraw = fused->q;
    a.q_bf16 = fused->bf16 ? 1 : 0;
    a.q_hadamard = fused->hadamard ? 1 : 0;
    a.q_c = fused->c;
  }
  hipError_t e = mxattn::launch_attention(a, (int)d, pnq ? 1 : 0, pr, s);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int mxattn_forward_quantized(const uint8_t* Qc, const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                             const uint8_t* VTc, const uint8_t* VTs, int64_t B, int64_t H, int64_t Nq,
                             int64_t Nkv, int64_t d, float softmax_scale, uint32_t pnq,
                             int32_t p_rule_kind, float p_qmax, void* O, int32_t out_dtype,
                             uint8_t* p_codes, uint8_t* p_scales, void* stream) {
  const char* who = "mxattn_forward_quantized";
  if (!Qc || !Qs || !Kc || !Ks || !VTc || !VTs || !O) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if ((p_codes == nullptr) != (p_scales == nullptr))
    return fail(MXATTN_E_INVALID, "%s: p_codes and p_scales must both be set or both be NULL", who);
  if (!aligned16(Qc) || !aligned16(Qs) || !aligned16(Kc) || !aligned16(Ks) || !aligned16(VTc) ||
      !aligned16(VTs) || !aligned16(O) || (p_codes && (!aligned16(p_codes) || !aligned16(p_scales))))
    return fail(MXATTN_E_INVALID, "%s: pointers must be 16-byte aligned", who);
  if (!elem_bytes(out_dtype)) return fail(MXATTN_E_INVALID, "%s: out_dtype must be MXATTN_F32 or MXATTN_BF16", who);
  if (int st = check_attn_shape(B, H, Nq, Nkv, d, softmax_scale, who)) return st;
  mxattn::Rule pr{};
  if (int st = make_rule(p_rule_kind, p_qmax, &pr, who)) return st;
  return attention_core(Qc, Qs, Kc, Ks, VTc, VTs, B, H, Nq, Nkv, d, softmax_scale, pnq, pr, O, out_dtype,
                        p_codes, p_scales, static_cast<hipStream_t>(stream), who);
}

int mxattn_arrange_scales(const uint8_t* Ks, const uint8_t* VTs, int64_t B, int64_t H, int64_t Nkv, int64_t d,
                          uint8_t* Ksa, uint8_t* VTsa, void* stream) {
  const char* who = "mxattn_arrange_scales";
  if (!Ks || !VTs || !Ksa || !VTsa) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if (!aligned16(Ks) || !aligned16(VTs) || !aligned16(Ksa) || !aligned16(VTsa))
    return fail(MXATTN_E_INVALID, "%s: pointers must be 16-byte aligned", who);
  if (int st = check_attn_shape(B, H, 1, Nkv, d, 1.0f, who)) return st;
  hipError_t e = mxattn::launch_arrange_scales(Ks, VTs, B * H, Nkv, round_up(Nkv, mxattn::kKvTile), (int)d, Ksa,
                                               VTsa, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int mxattn_forward_arranged(const uint8_t* Qc, const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ksa,
                            const uint8_t* VTc, const uint8_t* VTsa, int64_t B, int64_t H, int64_t Nq,
                            int64_t Nkv, int64_t d, float softmax_scale, uint32_t pnq, int32_t p_rule_kind,
                            float p_qmax, void* O, int32_t out_dtype, void* stream) {
  const char* who = "mxattn_forward_arranged";
  if (!Qc || !Qs || !Kc || !Ksa || !VTc || !VTsa || !O) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if (!aligned16(Qc) || !aligned16(Qs) || !aligned16(Kc) || !aligned16(Ksa) || !aligned16(VTc) ||
      !aligned16(VTsa) || !aligned16(O))
    return fail(MXATTN_E_INVALID, "%s: pointers must be 16-byte aligned", who);
  if (!elem_bytes(out_dtype)) return fail(MXATTN_E_INVALID, "%s: out_dtype must be MXATTN_F32 or MXATTN_BF16", who);
  if (int st = check_attn_shape(B, H, Nq, Nkv, d, softmax_scale, who)) return st;
  mxattn::Rule pr{};
  if (int st = make_rule(p_rule_kind, p_qmax, &pr, who)) return st;
  return attention_core(Qc, Qs, Kc, nullptr, VTc, nullptr, B, H, Nq, Nkv, d, softmax_scale, pnq, pr, O, out_dtype,
                        nullptr, nullptr, static_cast<hipStream_t>(stream), who, nullptr, Ksa, VTsa);
}

}  // extern "C"

namespace {

// Every check of mxattn_forward except those of the workspace: dtype, pointers, shape,
// rule, and the workspace layout the call needs (L).
int forward_checks(const void* Q, const void* K, const void* V, int32_t dtype, int64_t B, int64_t H, int64_t Nq,
                   int64_t Nkv, int64_t d, float softmax_scale, int32_t rule_kind, float qmax, const void* O,
                   const char* who, mxattn::Rule* rule, FwdLayout* L) {
  if (!elem_bytes(dtype)) return fail(MXATTN_E_INVALID, "%s: dtype must be MXATTN_F32 or MXATTN_BF16", who);
  if (!Q || !K || !V || !O) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(MXATTN_E_INVALID, "%s: pointers must be 16-byte aligned", who);
  if (int st = check_attn_shape(B, H, Nq, Nkv, d, softmax_scale, who)) return st;
  if (int st = make_rule(rule_kind, qmax, rule, who)) return st;
  if (!fwd_layout(B, H, Nq, Nkv, d, L)) return fail(MXATTN_E_INVALID, "%s: tensor too large", who);
  return MXATTN_OK;
}

}  // namespace

namespace mxattn {

int forward_arg_check(const void* Q, const void* K, const void* V, int32_t dtype, int64_t B, int64_t H, int64_t Nq,
                      int64_t Nkv, int64_t d, float softmax_scale, int32_t rule_kind, float qmax, const void* O,
                      const char* who, size_t* workspace_bytes) {
  Rule rule{};
  FwdLayout L;
  if (int st = forward_checks(Q, K, V, dtype, B, H, Nq, Nkv, d, softmax_scale, rule_kind, qmax, O, who, &rule, &L))
    return st;
  *workspace_bytes = L.total;
  return MXATTN_OK;
}

int set_error(int status, const char* message) { return fail(status, "%s", message); }

}  // namespace mxattn

extern "C" {

int mxattn_forward(const void* Q, const void* K, const void* V, int32_t dtype, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nkv, int64_t d, float softmax_scale, uint32_t hadamard,
                   uint32_t pnq, int32_t rule_kind, float qmax, void* O, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const char* who = "mxattn_forward";
  mxattn::Rule rule{};
  FwdLayout L;
  if (int st = forward_checks(Q, K, V, dtype, B, H, Nq, Nkv, d, softmax_scale, rule_kind, qmax, O, who, &rule, &L))
    return st;
  if (!workspace) return fail(MXATTN_E_INVALID, "%s: null pointer", who);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MXATTN_E_INVALID, "%s: workspace must be 256-byte aligned", who);
  if (workspace_bytes < L.total)
    return fail(MXATTN_E_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", who, workspace_bytes, L.total);
  const int eb = elem_bytes(dtype);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint8_t *kc = w + L.kc, *vc = w + L.vc, *ksa = w + L.ksa, *vsa = w + L.vsa;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t P = round_up(Nkv, mxattn::kKvTile);
  const float c = inv_sqrt_f32((int)d);
  hipError_t e;
  // K^ and V^T with their scales already in the attention kernel's operand order.  For a
  // small K and V (a few thousand tokens) both go in one launch, which saves a launch's
  // ramp (6 us of a 74 us step at 40 heads x 2048 tokens); for larger ones two launches
  // are faster, since in the joint kernel the token-axis quantiser runs at the Hadamard
  // quantiser's register count, three workgroups per CU instead of five.
  const bool joint = hadamard && B * H * Nkv * d * eb <= kJointQuantBytes;
  if (joint) {
    e = mxattn::launch_quant_kv(K, V, eb, (int)d, B * H, Nkv, P, kc, ksa, vc, vsa, rule, c, s);
  } else {
    if (hadamard)
      e = mxattn::launch_quant_hadamard(K, eb, (int)d, B * H * Nkv, kc, ksa, rule, c, nullptr, s, Nkv, P);
    else
      e = mxattn::launch_quant_last(K, eb, B * H * Nkv * d / 32, kc, ksa, rule, nullptr, s, (int)(d / 32), Nkv, P);
    if (e == hipSuccess) e = mxattn::launch_quant_rows(V, eb, B * H, Nkv, d, P, vc, vsa, rule, nullptr, s, true);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  // Q is read once per query tile: the attention kernel rotates and quantises it itself
  const QuantQ fused{Q, eb == 2, hadamard != 0, c};
  return attention_core(nullptr, nullptr, kc, nullptr, vc, nullptr, B, H, Nq, Nkv, d, softmax_scale, pnq, rule, O,
                        dtype, nullptr, nullptr, s, who, &fused, ksa, vsa);
}

}  // extern "C"
