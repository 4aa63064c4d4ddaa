// Host-only driver of the C ABI's argument validation, built with
// AddressSanitizer over the library's host code (tests/test_abi_asan.py).
// Every call below is rejected before any device work: null, misaligned or
// too-small arguments, invalid problems, unsupported combinations.  The driver
// checks each status and prints "ok" at the end; AddressSanitizer reports any
// out-of-bounds or use-after-free access in the validation code itself.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/dspark.h"
#include "../../include/dspark_instr.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

static dspark_problem problem(int B, int K, int V, int r, int d, int logits, int weights, int hidden, float T) {
  dspark_problem p;
  memset(&p, 0, sizeof(p));
  p.B = B;
  p.K = K;
  p.V = V;
  p.r = r;
  p.d = d;
  p.logits_dtype = logits;
  p.weight_dtype = weights;
  p.hidden_dtype = hidden;
  p.sampling_temp = T;
  p.seed = 7;
  return p;
}

int main() {
  const dspark_problem ok = problem(256, 16, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f);
  // fake device addresses: validation never dereferences them
  void* f[24];
  for (int i = 0; i < 24; ++i) f[i] = (void*)(uintptr_t)(0x100000u * (i + 1));
  void* mis = (void*)(uintptr_t)0x100008u;  // 8-byte aligned, not 16
  void* ws = (void*)(uintptr_t)0x40000000u;
  const size_t need = dspark_workspace_bytes(&ok);
  if (need == 0) {
    printf("FAIL workspace size of the headline problem\n");
    return 1;
  }

  // problems
  const dspark_problem bad[] = {
      problem(0, 16, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 0, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 65, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 16, 1004, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 16, 151936, 0, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 16, 151936, 256, 0, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f),
      problem(256, 16, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 0.0f),
      problem(256, 16, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, -1.0f),
  };
  for (const dspark_problem& p : bad) {
    expect("workspace_bytes(bad)", (int)dspark_workspace_bytes(&p), 0);
    expect("draft(bad)", dspark_draft(&p, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f, (const float*)f[5],
                                      (const int32_t*)f[6], (int32_t*)f[7], (float*)f[8], (float*)f[9],
                                      (float*)f[10], (float*)f[11], ws, need, nullptr),
           DSPARK_E_INVALID);
    expect("schedule(bad)", dspark_schedule(&p, (const float*)f[0], (const float*)f[1], (int32_t*)f[2],
                                            (int32_t*)f[3], ws, need, nullptr),
           DSPARK_E_INVALID);
  }
  const dspark_problem dt = problem(256, 16, 151936, 256, 4096, 7, DSPARK_BF16, DSPARK_BF16, 1.0f);
  expect("draft(dtype)", dspark_draft(&dt, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f, (const float*)f[5],
                                      (const int32_t*)f[6], (int32_t*)f[7], (float*)f[8], (float*)f[9],
                                      (float*)f[10], (float*)f[11], ws, need, nullptr),
         DSPARK_E_DTYPE);
  const dspark_problem r48 = problem(256, 16, 151936, 48, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f);
  expect("workspace_bytes(r48)", (int)dspark_workspace_bytes(&r48), 0);

  // pointers
  expect("draft(null P)", dspark_draft(nullptr, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f,
                                       (const float*)f[5], (const int32_t*)f[6], (int32_t*)f[7], (float*)f[8],
                                       (float*)f[9], (float*)f[10], (float*)f[11], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("draft(null Z)", dspark_draft(&ok, nullptr, f[1], f[2], f[3], (const float*)f[4], 0.f, (const float*)f[5],
                                       (const int32_t*)f[6], (int32_t*)f[7], (float*)f[8], (float*)f[9],
                                       (float*)f[10], (float*)f[11], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("draft(misaligned E)", dspark_draft(&ok, f[0], mis, f[2], f[3], (const float*)f[4], 0.f,
                                             (const float*)f[5], (const int32_t*)f[6], (int32_t*)f[7],
                                             (float*)f[8], (float*)f[9], (float*)f[10], (float*)f[11], ws, need,
                                             nullptr),
         DSPARK_E_POINTER);
  expect("draft(small workspace)", dspark_draft(&ok, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f,
                                                (const float*)f[5], (const int32_t*)f[6], (int32_t*)f[7],
                                                (float*)f[8], (float*)f[9], (float*)f[10], (float*)f[11], ws,
                                                need - 256, nullptr),
         DSPARK_E_WORKSPACE);
  expect("draft(null workspace)", dspark_draft(&ok, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f,
                                               (const float*)f[5], (const int32_t*)f[6], (int32_t*)f[7],
                                               (float*)f[8], (float*)f[9], (float*)f[10], (float*)f[11], nullptr,
                                               need, nullptr),
         DSPARK_E_WORKSPACE);
  expect("draft_timed(bad path)",
         dspark_draft_timed(&ok, f[0], f[1], f[2], f[3], (const float*)f[4], 0.f, (const float*)f[5],
                            (const int32_t*)f[6], (int32_t*)f[7], (float*)f[8], (float*)f[9], (float*)f[10],
                            (float*)f[11], ws, need, nullptr, nullptr, 0, 9),
         DSPARK_E_INVALID);
  expect("schedule(null T)", dspark_schedule(&ok, (const float*)f[0], nullptr, (int32_t*)f[2], (int32_t*)f[3], ws,
                                             need, nullptr),
         DSPARK_E_POINTER);
  const dspark_problem big = problem(2048, 32, 151936, 256, 4096, DSPARK_BF16, DSPARK_BF16, DSPARK_BF16, 1.0f);
  expect("schedule_noalloc(65,536 candidates)",
         dspark_schedule_noalloc(&big, (const float*)f[0], (const float*)f[1], (int32_t*)f[2], (int32_t*)f[3],
                                 nullptr),
         DSPARK_E_WORKSPACE);
  expect("schedule_fixed(gamma > K)", dspark_schedule_fixed(&ok, 17, (int32_t*)f[2], (int32_t*)f[3], nullptr),
         DSPARK_E_INVALID);
  expect("schedule_threshold(nan)", dspark_schedule_threshold(&ok, (const float*)f[0], __builtin_nanf(""),
                                                              (int32_t*)f[2], (int32_t*)f[3], nullptr),
         DSPARK_E_INVALID);
  expect("schedule_async(null lag)", dspark_schedule_async(&ok, nullptr, (const float*)f[1], (const float*)f[2],
                                                           (int32_t*)f[3], (int32_t*)f[4], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("verify(null target)", dspark_verify(&ok, nullptr, f[1], f[2], f[3], (const int32_t*)f[4],
                                              (const int32_t*)f[5], (const float*)f[6], (const float*)f[7],
                                              (const int32_t*)f[8], (int32_t*)f[9], (int32_t*)f[10],
                                              (int32_t*)f[11], (float*)f[12], (float*)f[13], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("verify(misaligned Wt)", dspark_verify(&ok, f[0], f[1], f[2], mis, (const int32_t*)f[4],
                                                (const int32_t*)f[5], (const float*)f[6], (const float*)f[7],
                                                (const int32_t*)f[8], (int32_t*)f[9], (int32_t*)f[10],
                                                (int32_t*)f[11], (float*)f[12], (float*)f[13], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("verify_rnn(null state)", dspark_verify_rnn(&ok, f[0], f[1], f[2], f[3], (const int32_t*)f[4],
                                                     (const int32_t*)f[5], (const float*)f[6], (const float*)f[7],
                                                     nullptr, (const int32_t*)f[8], (int32_t*)f[9],
                                                     (int32_t*)f[10], (int32_t*)f[11], (float*)f[12],
                                                     (float*)f[13], ws, need, nullptr),
         DSPARK_E_POINTER);
  expect("sts_fit(bins)", dspark_sts_fit(10, 4, (const float*)f[0], (const int32_t*)f[1], (const int32_t*)f[2],
                                         (const double*)f[3], 8, 17, (double*)f[4], (int32_t*)f[5],
                                         (double*)f[6], (double*)f[7], ws, 1 << 20, nullptr),
         DSPARK_E_INVALID);
  expect("probe_draws(n < 0)", dspark_probe_draws(1, (const uint32_t*)f[0], -1, (uint32_t*)f[1], nullptr, 0,
                                                  nullptr, nullptr, nullptr),
         DSPARK_E_INVALID);
  expect("draft_path(bad)", dspark_draft_path(&bad[0]), DSPARK_E_INVALID);
  // status strings: every code and an unknown one
  for (int c = -8; c <= 1; ++c)
    if (!dspark_status_string(c) || !dspark_status_string(c)[0]) {
      printf("FAIL status_string(%d)\n", c);
      ++failures;
    }
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
