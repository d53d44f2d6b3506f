// mxattn_forward_noalloc: mxattn_forward with its workspace in a library-owned device
// array, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this translation unit.  In host code its name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what the kernels
// receive.  Every call on one GPU uses that GPU's copy: calls that overlap in time on
// one GPU race.  Nothing needs clearing between calls: the pipeline rewrites every
// workspace byte whose value reaches the output (K^, the padded V^T, their scales in the
// attention kernel's operand order) before reading it; the only bytes it reads without
// rewriting are the scales of the key slots past the last key, which feed logits the
// kernel then masks, and at d = 64 the operand bytes that no MFMA selects.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "launch.h"
#include "mxattn.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MXATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per device: the address of that device's `scratch`

// The current device's copy of `scratch` (looked up on the device's first call).
int scratch_address(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  char msg[256];
  if (e != hipSuccess) {
    std::snprintf(msg, sizeof msg, "%s: hipGetDevice failed: HIP error %d (%s)", who, (int)e, hipGetErrorString(e));
    return mxattn::set_error(MXATTN_E_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(msg, sizeof msg, "%s: device %d is beyond the %d devices this entry supports", who, dev,
                  kMaxDevices);
    return mxattn::set_error(MXATTN_E_UNSUPPORTED, msg);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      std::snprintf(msg, sizeof msg, "%s: hipGetSymbolAddress of the scratch array failed on device %d: HIP error "
                    "%d (%s)", who, dev, (int)e, hipGetErrorString(e));
      return mxattn::set_error(MXATTN_E_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXATTN_OK;
}

}  // namespace

extern "C" int mxattn_forward_noalloc(const void* Q, const void* K, const void* V, int32_t dtype, int64_t B,
                                      int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float softmax_scale,
                                      uint32_t hadamard, uint32_t pnq, int32_t rule_kind, float qmax, void* O,
                                      void* stream) {
  const char* who = "mxattn_forward_noalloc";
  size_t need = 0;
  if (int st = mxattn::forward_arg_check(Q, K, V, dtype, B, H, Nq, Nkv, d, softmax_scale, rule_kind, qmax, O, who,
                                         &need))
    return st;
  if (need > MXATTN_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "%s: this call needs %zu bytes of scratch; the library's array holds %zu "
                  "(use mxattn_forward with a workspace)", who, need, (size_t)MXATTN_NOALLOC_SCRATCH_BYTES);
    return mxattn::set_error(MXATTN_E_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (int st = scratch_address(&ws, who)) return st;
  return mxattn_forward(Q, K, V, dtype, B, H, Nq, Nkv, d, softmax_scale, hadamard, pnq, rule_kind, qmax, O, ws,
                        MXATTN_NOALLOC_SCRATCH_BYTES, stream);
}
