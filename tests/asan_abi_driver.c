/* Host-only exercise of every argument check of the C ABI, built with AddressSanitizer
 * (tests/test_asan_host.py).  Device pointers are fake aligned addresses that a call
 * must never dereference: every call here fails validation before any HIP call. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mxattn.h"

#define FAKE ((void*)(uintptr_t)(1u << 20))
#define FAKE8 ((uint8_t*)(uintptr_t)(1u << 20))
#define MIS ((void*)(uintptr_t)((1u << 20) + 4))

static int failures = 0;

static void expect(int got, int want, const char* what) {
  const char* msg = mxattn_last_error();
  if (got != want || (want != MXATTN_OK && (msg == NULL || strlen(msg) == 0))) {
    printf("FAIL %s: status %d (want %d), message '%s'\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

int main(void) {
  /* constants and sizes, including overflowing ones */
  if (mxattn_kv_tile() != 128) ++failures;
  if (mxattn_padded_tokens(1) != 128 || mxattn_padded_tokens(-5) != -1) ++failures;
  if (mxattn_forward_workspace_bytes(1, 40, 75600, 75600, 128) == 0) ++failures;
  if (mxattn_forward_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, 128) != 0) ++failures;
  if (mxattn_forward_workspace_bytes(1, 1, 1, 1, 96) != 0) ++failures;

  /* quantizer */
  expect(mxattn_quantize(NULL, MXATTN_BF16, 1, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8,
                         NULL), MXATTN_E_INVALID, "quantize null x");
  expect(mxattn_quantize(FAKE, 7, 1, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8, NULL),
         MXATTN_E_INVALID, "quantize dtype");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 1, 32, 100, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8,
                         NULL), MXATTN_E_INVALID, "quantize cols % 32");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 1, 32, 96, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 1, FAKE8, FAKE8,
                         NULL), MXATTN_E_UNSUPPORTED, "quantize hadamard cols");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 1, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_CEIL, 3.5f, 0, FAKE8,
                         FAKE8, NULL), MXATTN_E_INVALID, "quantize qmax");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 1, 32, 128, 9, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8, NULL),
         MXATTN_E_INVALID, "quantize axis");
  expect(mxattn_quantize(MIS, MXATTN_F32, 1, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8,
                         NULL), MXATTN_E_INVALID, "quantize misaligned");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 0, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, FAKE8, FAKE8,
                         NULL), MXATTN_E_INVALID, "quantize empty");
  expect(mxattn_quantize(FAKE, MXATTN_F32, 1, 32, 128, MXATTN_AXIS_ROWS, MXATTN_RULE_UOS, 0.f, 1, FAKE8, FAKE8,
                         NULL), MXATTN_E_INVALID, "quantize rows with rotation");
  expect(mxattn_quant_error(FAKE, MXATTN_F32, 1, 32, 128, MXATTN_AXIS_LAST, MXATTN_RULE_UOS, 0.f, 0, NULL, NULL),
         MXATTN_E_INVALID, "quant_error null sums");

  /* forward */
  const size_t ws = mxattn_forward_workspace_bytes(1, 2, 256, 256, 64);
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, 256, 256, 64, 0.125f, 1, 1, MXATTN_RULE_UOS, 0.f, FAKE,
                        FAKE, ws - 1, NULL), MXATTN_E_WORKSPACE, "forward small workspace");
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, 256, 256, 96, 0.125f, 1, 1, MXATTN_RULE_UOS, 0.f, FAKE,
                        FAKE, ws, NULL), MXATTN_E_UNSUPPORTED, "forward d");
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, 0, 256, 64, 0.125f, 1, 1, MXATTN_RULE_UOS, 0.f, FAKE,
                        FAKE, ws, NULL), MXATTN_E_INVALID, "forward Nq = 0");
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, 256, 256, 64, -1.f, 1, 1, MXATTN_RULE_UOS, 0.f, FAKE,
                        FAKE, ws, NULL), MXATTN_E_INVALID, "forward scale");
  expect(mxattn_forward(FAKE, FAKE, NULL, MXATTN_F32, 1, 2, 256, 256, 64, 0.125f, 1, 1, MXATTN_RULE_UOS, 0.f,
                        FAKE, FAKE, ws, NULL), MXATTN_E_INVALID, "forward null V");
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, 256, 256, 64, 0.125f, 1, 1, MXATTN_RULE_UOS, 0.f, FAKE,
                        MIS, ws, NULL), MXATTN_E_INVALID, "forward workspace alignment");
  expect(mxattn_forward(FAKE, FAKE, FAKE, MXATTN_F32, 1, 2, (int64_t)1 << 25, 256, 64, 0.125f, 1, 1,
                        MXATTN_RULE_UOS, 0.f, FAKE, FAKE, ws, NULL), MXATTN_E_INVALID, "forward too many tokens");
  expect(mxattn_forward_quantized(FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, 1, 2, 256, 256, 64, 0.125f, 1,
                                  MXATTN_RULE_UOS, 0.f, FAKE, MXATTN_F32, FAKE8, NULL, NULL),
         MXATTN_E_INVALID, "forward_quantized half a dump");
  expect(mxattn_forward_quantized(FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, 1, 2, 256, 256, 64, 0.125f, 1,
                                  MXATTN_RULE_OCP, 0.f, FAKE, 5, NULL, NULL, NULL),
         MXATTN_E_INVALID, "forward_quantized out dtype");

  expect(mxattn_arrange_scales(FAKE8, FAKE8, 1, 2, 300, 128, NULL, FAKE8, NULL), MXATTN_E_INVALID,
         "arrange null output");
  expect(mxattn_arrange_scales(FAKE8, (const uint8_t*)MIS, 1, 2, 300, 128, FAKE8, FAKE8, NULL), MXATTN_E_INVALID,
         "arrange misaligned");
  expect(mxattn_arrange_scales(FAKE8, FAKE8, 1, 2, 300, 80, FAKE8, FAKE8, NULL), MXATTN_E_UNSUPPORTED,
         "arrange d");
  expect(mxattn_forward_arranged(FAKE8, FAKE8, FAKE8, NULL, FAKE8, FAKE8, 1, 2, 256, 256, 64, 0.125f, 1,
                                 MXATTN_RULE_UOS, 0.f, FAKE, MXATTN_F32, NULL), MXATTN_E_INVALID,
         "forward_arranged null scales");
  expect(mxattn_forward_arranged(FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, FAKE8, 1, 2, 256, 256, 64, 0.125f, 1, 9, 0.f,
                                 FAKE, MXATTN_F32, NULL), MXATTN_E_INVALID, "forward_arranged rule");

  /* a long message must not overflow the thread-local buffer */
  for (int i = 0; i < 1000; ++i)
    (void)mxattn_quantize(FAKE, 1000 + i, 1, 32, 128, 0, 0, 0.f, 0, FAKE8, FAKE8, NULL);
  printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
