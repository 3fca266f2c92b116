/* Host-side exercise of libkvc's C ABI for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code.  Every call made here either is host-only
 * (workspace sizes, packed capacities, pilot budgets, status strings) or fails argument
 * validation before any device is touched, so the driver runs on a machine without a GPU and
 * never launches a kernel.  It returns 0 when every call gave the expected status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvc.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t rand_range(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

static kvc_layer_desc random_desc(void) {
  kvc_layer_desc d;
  memset(&d, 0, sizeof d);
  const int g_choices[] = {1, 2, 3, 4, 7, 8, 16};
  d.n_kv_heads = (int32_t)rand_range(1, 12);
  d.n_q_heads = d.n_kv_heads * g_choices[rand_range(0, 6)];
  d.head_dim = rand_range(0, 1) ? 64 : 128;
  d.causal = (int32_t)rand_range(0, 1);
  d.n_keys = rand_range(1, 1 << 20);
  d.n_queries = rand_range(1, d.n_keys < 70000 ? d.n_keys : 70000);
  d.softmax_scale = 0.f;
  return d;
}

int main(void) {
  char* fake = (char*)(uintptr_t)0x100000;   /* aligned, never dereferenced on these paths */
  /* workspace sizes and packed capacities over many layers */
  for (int it = 0; it < 3000; ++it) {
    kvc_layer_desc d = random_desc();
    for (int op = 0; op < 7; ++op)
      for (int mode = 0; mode < 3; ++mode) {
        size_t b = kvc_workspace_size(op, &d, op == 6 ? (int32_t)rand_range(1, 300) : mode);
        EXPECT(b < ((size_t)1 << 56));   /* large layers need large workspaces; no wrap-around */
      }
    size_t caps[KVC_PK_NBUF];
    EXPECT(kvc_packed_capacity(&d, 32, caps) == KVC_OK);
    EXPECT(kvc_packed_capacity(&d, 16, caps) != KVC_OK);
  }
  /* invalid descriptors are refused by every call */
  kvc_layer_desc bad = random_desc();
  bad.n_q_heads = bad.n_kv_heads * 3 + 1;
  if (bad.n_q_heads % bad.n_kv_heads == 0) bad.n_q_heads += 1;
  EXPECT(kvc_workspace_size(0, &bad, 0) == 0);
  EXPECT(kvc_row_lse(&bad, fake, fake, (float*)fake, fake, 1 << 20, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_row_lse(NULL, fake, fake, (float*)fake, fake, 1 << 20, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(strlen(kvc_last_error()) > 0);
  kvc_layer_desc ok = random_desc();
  /* NULL and misaligned data pointers are refused before any device work */
  EXPECT(kvc_row_lse(&ok, NULL, fake, (float*)fake, fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_row_lse(&ok, fake + 2, fake, (float*)fake, fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_row_lse_noalloc(&ok, fake, fake + 8, (float*)fake, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_score_tokens(&ok, (kvc_score_mode)5, fake, fake, (float*)fake, NULL, (float*)fake, fake, 1, NULL) ==
         KVC_ERR_INVALID_ARG);
  EXPECT(kvc_score_tokens(&ok, KVC_SCORE_MAX, fake, fake, (float*)fake, NULL, (float*)fake, fake, (size_t)1 << 40,
                          NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_channel_weights(&ok, fake, fake, NULL, fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_row_lse(&ok, fake, fake, (float*)fake, fake, 0, NULL) == KVC_ERR_WORKSPACE);
  EXPECT(kvc_allocate_bits(&ok, KVC_ALLOC_V_TOKENS, (float*)fake, NULL, NULL, -1.0, 0.0, 16, (uint8_t*)fake, NULL,
                           fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_allocate_bits(&ok, KVC_ALLOC_V_TOKENS, (float*)fake, NULL, NULL, NAN, 0.0, 16, (uint8_t*)fake, NULL,
                           fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_allocate_bits(&ok, KVC_ALLOC_TOPK, (float*)fake, NULL, NULL, 0.0, 1.5, 16, (uint8_t*)fake, NULL, fake,
                           (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_allocate_bits(&ok, KVC_ALLOC_TOPK, (float*)fake, NULL, NULL, 0.0, 0.5, 3, (uint8_t*)fake, NULL, fake,
                           (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_allocate_bits(&ok, KVC_ALLOC_K_CHANNELS, (float*)fake, NULL, NULL, 2.0, 0.0, 16, (uint8_t*)fake, NULL,
                           fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_keep_threshold(&ok, (float*)fake, NAN, 128, 16, (uint8_t*)fake, NULL, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_keep_threshold(&ok, (float*)fake, 1.f, -1, 16, (uint8_t*)fake, NULL, NULL) == KVC_ERR_INVALID_ARG);
  kvc_packed_cache pc;
  memset(&pc, 0, sizeof pc);
  EXPECT(kvc_quantize_pack(&ok, fake, fake, (uint8_t*)fake, (uint8_t*)fake, 32, &pc, fake, (size_t)1 << 40, NULL) ==
         KVC_ERR_INVALID_ARG);
  EXPECT(kvc_quantize_pack(&ok, fake, fake, (uint8_t*)fake, (uint8_t*)fake, 64, &pc, fake, (size_t)1 << 40, NULL) !=
         KVC_OK);
  EXPECT(kvc_compressed_attend(&ok, fake, NULL, (float*)fake, (float*)fake, fake, (size_t)1 << 40, NULL) ==
         KVC_ERR_INVALID_ARG);
  EXPECT(kvc_compressed_attend_append(&ok, fake, &pc, fake, fake, -3, (float*)fake, (float*)fake, fake,
                                      (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_fidelity_terms(&ok, NULL, (float*)fake, (float*)fake, (float*)fake, (double*)fake, NULL) ==
         KVC_ERR_INVALID_ARG);
  EXPECT(kvc_ridge_value_fit(&ok, 0, fake, fake, fake, (float*)fake, 0.1, (float*)fake, fake, (size_t)1 << 40,
                             NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_ridge_value_fit(&ok, 1, fake, fake, fake, (float*)fake, -1.0, (float*)fake, fake, (size_t)1 << 40,
                             NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_get_device_status(NULL, NULL, NULL) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_allocate_bits(&ok, (kvc_alloc_stage)-7, (float*)fake, NULL, NULL, 1.0, 0.0, 16, (uint8_t*)fake, NULL,
                           fake, (size_t)1 << 40, NULL) == KVC_ERR_INVALID_ARG);
  /* pilot budgets (host arithmetic): budgets add up to the total and honour the floor */
  for (int it = 0; it < 20000; ++it) {
    const int n = (int)rand_range(1, 64);
    double mse[64];
    int64_t out[64];
    for (int i = 0; i < n; ++i) {
      const int kind = (int)rand_range(0, 9);
      mse[i] = kind == 0 ? 0.0 : exp((double)rand_range(-40000, 40000) / 1000.0);
    }
    const int64_t floor_each = rand_range(0, 1000);
    const int64_t total = n * floor_each + rand_range(0, (int64_t)1 << 40);
    EXPECT(kvc_pilot_budgets(mse, n, total, floor_each, out) == KVC_OK);
    int64_t sum = 0;
    for (int i = 0; i < n; ++i) {
      EXPECT(out[i] >= floor_each);
      sum += out[i];
    }
    EXPECT(sum == total);
  }
  double neg = -1.0;
  int64_t one_out;
  EXPECT(kvc_pilot_budgets(&neg, 1, 10, 0, &one_out) == KVC_ERR_INVALID_ARG);
  EXPECT(kvc_pilot_budgets(NULL, 1, 10, 0, &one_out) == KVC_ERR_INVALID_ARG);
  for (int st = 0; st < 9; ++st) EXPECT(kvc_status_string((kvc_status)st) != NULL);
  EXPECT(strncmp(kvc_version(), "kvc ", 4) == 0);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host sanitizer driver: all expectations met\n");
  return 0;
}
