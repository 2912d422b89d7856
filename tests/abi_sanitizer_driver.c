/* Host-side rejection paths of the C ABI (include/tara.h), called from C.
 * tests/test_abi_sanitized.py builds this driver together with the library
 * sources, host code instrumented with AddressSanitizer and
 * UndefinedBehaviorSanitizer, and runs it on a machine without a GPU: every
 * call below fails its host checks (or is an empty call) before any device
 * work, so no pointer here is ever dereferenced on a device. Prints one line
 * per check and "ALL OK" at the end; exits 1 on the first wrong status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tara.h"

#define FAKE ((void*)0x10000)

static int failures = 0;

static void expect(const char* what, int got, int want) {
  printf("%-58s status %3d (want %3d) %s\n", what, got, want, got == want ? "ok" : "WRONG");
  if (got != want) failures++;
}

static int call(const tara_params_t* p, int dt, int B, int H, int N, int D, void* q, void* seg,
                const int64_t* str, void* ws, size_t ws_bytes) {
  int64_t s[3];
  if (str) memcpy(s, str, sizeof s);
  else { s[0] = (int64_t)H * N * D; s[1] = (int64_t)N * D; s[2] = D; }
  return tara_attn_fwd(q, FAKE, FAKE, FAKE, (float*)FAKE, dt, B, H, N, D, s, s, s, s, (const uint8_t*)seg,
                       (const float*)FAKE, (const int16_t*)FAKE, NULL, p, ws, ws_bytes, NULL);
}

static int call_na(const tara_params_t* p, int N, void* q) {
  const int64_t s[3] = {2 * (int64_t)N * 128, (int64_t)N * 128, 128};
  return tara_attn_fwd_noalloc(q, FAKE, FAKE, FAKE, (float*)FAKE, TARA_BF16, 1, 2, N, 128, s, s, s, s,
                               (const uint8_t*)FAKE, (const float*)FAKE, (const int16_t*)FAKE, NULL, p, NULL);
}

int main(void) {
  tara_params_t p, d;
  tara_params_default(&d);
  const size_t big = (size_t)1 << 40;

  expect("params NULL", call(NULL, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_NULL_POINTER);
  expect("dtype 5", call(&d, 5, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_UNSUPPORTED_DTYPE);
  expect("head dim 96", call(&d, TARA_BF16, 1, 2, 100, 96, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_UNSUPPORTED_HEAD_DIM);
  expect("N = -1", call(&d, TARA_BF16, 1, 2, -1, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_SHAPE);
  expect("B * H > 65535", call(&d, TARA_BF16, 300, 300, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_SHAPE);
  expect("q NULL", call(&d, TARA_BF16, 1, 2, 100, 128, NULL, FAKE, NULL, FAKE, big), TARA_ERR_NULL_POINTER);
  expect("seg_type NULL", call(&d, TARA_BF16, 1, 2, 100, 128, FAKE, NULL, NULL, FAKE, big), TARA_ERR_NULL_POINTER);
  expect("q base not 16-byte aligned",
         call(&d, TARA_BF16, 1, 2, 100, 128, (char*)FAKE + 8, FAKE, NULL, FAKE, big), TARA_ERR_BAD_STRIDE);
  const int64_t bad_row[3] = {1000 * 128, 100 * 128, 130};
  expect("row stride not a multiple of 8", call(&d, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, bad_row, FAKE, big),
         TARA_ERR_BAD_STRIDE);
  expect("workspace too small", call(&d, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, 10), TARA_ERR_WORKSPACE);
  expect("workspace NULL", call(&d, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, NULL, big), TARA_ERR_WORKSPACE);
  expect("workspace not 256-byte aligned",
         call(&d, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, (char*)FAKE + 64, big), TARA_ERR_WORKSPACE);
  const int n20 = 1 << 20;
  const int64_t bnhd8[3] = {(int64_t)n20 * 8 * 128, 128, 8 * 128};
  expect("bf16 tile offsets past 2^31", call(&d, TARA_BF16, 1, 8, n20, 128, FAKE, FAKE, bnhd8, FAKE, 10),
         TARA_ERR_BAD_STRIDE);

  float bad_floats[] = {0.0f, -1.0f, NAN, INFINITY};
  for (int i = 0; i < 4; ++i) {
    p = d;
    p.falloff = bad_floats[i];
    char what[64];
    snprintf(what, sizeof what, "falloff %g", bad_floats[i]);
    expect(what, call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  }
  p = d; p.window = -0.1f;
  expect("window < 0", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.cap = INFINITY;
  expect("cap infinite", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.binding_enabled = 1; p.num_pictures = 2; p.picture_gain[0][1] = 0.0f;
  expect("gain 0", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.binding_enabled = 1; p.num_pictures = 17;
  expect("17 pictures", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.binding_enabled = 1; p.num_pictures = 1; p.num_bindings = 5;
  expect("5 bindings", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.mode = TARA_MODE_PARTITIONED; p.num_partitions = 65;
  expect("65 partitions", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  const int32_t descending[3] = {0, 60, 50};
  p = d; p.mode = TARA_MODE_PARTITIONED; p.num_partitions = 2; p.partition_bounds = descending;
  expect("partition bounds descending", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big),
         TARA_ERR_BAD_PARAM);
  p = d; p.mode = 7;
  expect("mode 7", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_PARAM);
  p = d; p.qk8 = 1; p.mode = TARA_MODE_THREE_TERM;
  expect("qk8 in three-term mode", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big),
         TARA_ERR_BAD_PARAM);
  p = d; p.mode = TARA_MODE_FRAME_LOOP; p.num_partitions = 101;
  expect("frame loop: more ranges than rows", call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big),
         TARA_ERR_BAD_PARAM);
  p = d; p.mode = TARA_MODE_THREE_TERM;
  expect("three-term beyond 2^20 tokens",
         call(&p, TARA_BF16, 1, 1, (1 << 20) + 64, 128, FAKE, FAKE, NULL, FAKE, big), TARA_ERR_BAD_SHAPE);

  expect("empty call N = 0", call(&d, TARA_BF16, 1, 2, 0, 128, NULL, NULL, NULL, NULL, 0), TARA_OK);
  tara_run_info_t info;
  expect("run info of the empty call", tara_get_last_run_info(&info), TARA_OK);
  expect("  ... launches", info.launches, 0);
  expect("run info NULL", tara_get_last_run_info(NULL), TARA_ERR_NULL_POINTER);

  expect("no-alloc: params NULL", call_na(NULL, 100, FAKE), TARA_ERR_NULL_POINTER);
  expect("no-alloc: q NULL", call_na(&d, 100, NULL), TARA_ERR_NULL_POINTER);
  p = d; p.falloff = 0.0f;
  expect("no-alloc: falloff 0", call_na(&p, 100, FAKE), TARA_ERR_BAD_PARAM);
  expect("no-alloc: empty call", call_na(&d, 0, NULL), TARA_OK);
  p = d; p.mode = TARA_MODE_DENSE_BIAS;
  expect("no-alloc: one head beyond the array", call_na(&p, 8192, FAKE), TARA_ERR_WORKSPACE);

  float tf = 0.0f;
  expect("probe: tflops NULL", tara_probe_mfma_bf16(100, 1, NULL, NULL), TARA_ERR_NULL_POINTER);
  expect("probe: 0 iterations", tara_probe_mfma_bf16(0, 1, &tf, NULL), TARA_ERR_BAD_PARAM);
  expect("probe: operand kind 2", tara_probe_mfma_bf16(100, 2, &tf, NULL), TARA_ERR_BAD_PARAM);
  int count = -1;
  expect("timing read, nothing recorded", tara_timing_read(NULL, 0, &count), TARA_OK);
  expect("  ... count", count, 0);
  expect("timing read, count NULL", tara_timing_read(NULL, 0, NULL), TARA_ERR_NULL_POINTER);

  p = d;
  p.mode = TARA_MODE_PARTITIONED; p.num_partitions = 0;
  expect("workspace bytes of a rejected shape", tara_workspace_bytes(TARA_BF16, 1, 2, 100, 128, &p) == (size_t)-1, 1);
  expect("workspace bytes of an empty call", (int)tara_workspace_bytes(TARA_BF16, 0, 2, 100, 128, &d), 0);
  for (int st = 1; st >= -10; --st) {
    const char* m = tara_status_string(st);
    expect("status string is text", m != NULL && strlen(m) > 0, 1);
  }
  call(&p, TARA_BF16, 1, 2, 100, 128, FAKE, FAKE, NULL, FAKE, big);
  expect("last error names the problem", strstr(tara_last_error(), "num_partitions") != NULL, 1);
  if (failures) {
    printf("%d WRONG\n", failures);
    return 1;
  }
  printf("ALL OK\n");
  return 0;
}
