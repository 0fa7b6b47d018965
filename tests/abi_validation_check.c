/*
 * Host-side argument validation of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_abi_sanitized.py from the
 * library's sources, host code only).  Every call below is invalid in some
 * way and must be refused with its status code before any HIP call, so the
 * driver needs no GPU.  The sizes helpers are called on valid and invalid
 * dims.  A sanitizer report, or a status other than the one expected, fails
 * the run.
 */
#include <stdint.h>
#include <stdio.h>

#include "moe.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL: %s returned %d, expected %d (%s)\n", what, got, want,
            moe_strerror(got));
    ++failures;
  }
}

int main(void) {
  const moe_dims glm = {6144, 2048, 256, 8, 64};
  const moe_dims perrow = {6144, 2048, 256, 8, 0};
  const moe_dims bad_group = {6144, 2048, 256, 8, 32};
  const moe_dims bad_d = {6100, 2048, 256, 8, 64};
  const moe_dims bad_k = {6144, 2048, 256, 33, 64};
  const moe_dims k_over_e = {256, 128, 4, 8, 64};
  /* aligned, never dereferenced */
  void* const p = (void*)(uintptr_t)(1u << 20);
  float* const fp = (float*)p;
  int32_t* const ip = (int32_t*)p;
  const void* const* tab = (const void* const*)p;
  const size_t ws1 = moe_workspace_bytes(&glm, 1);

  if (moe_expert_blob_bytes(&glm) != 20054016u) ++failures;
  if (moe_expert_blob_bytes(&perrow) != 18894848u) ++failures;
  if (moe_expert_blob_bytes(&bad_group) != 0 || moe_expert_blob_bytes(NULL) != 0) ++failures;
  if (ws1 == 0 || moe_workspace_bytes(&glm, 0) != 0 || moe_workspace_bytes(&bad_d, 4) != 0)
    ++failures;
  moe_routing_offsets ro;
  expect(moe_workspace_routing(&glm, 8, &ro), MOE_OK, "routing offsets");
  expect(moe_workspace_routing(&glm, 0, &ro), MOE_EINVAL, "routing offsets T = 0");
  expect(moe_workspace_routing(&bad_k, 1, &ro), MOE_EUNSUPPORTED, "routing offsets k = 33");
  if (moe_cache_state_bytes(&glm, 12) == 0 || moe_cache_state_bytes(&glm, 0) != 0) ++failures;
  for (int c = -6; c <= 1; ++c) (void)moe_strerror(c);

  expect(moe_route(NULL, p, MOE_F32, 1, fp, NULL, ip, fp, p, ws1, NULL), MOE_EINVAL, "route dims");
  expect(moe_route(&bad_group, p, MOE_F32, 1, fp, NULL, ip, fp, p, ws1, NULL), MOE_EUNSUPPORTED,
         "route group");
  expect(moe_route(&k_over_e, p, MOE_F32, 1, fp, NULL, ip, fp, p, ws1, NULL), MOE_EINVAL,
         "route k > E");
  expect(moe_route(&glm, p, 7, 1, fp, NULL, ip, fp, p, ws1, NULL), MOE_EUNSUPPORTED, "route dtype");
  expect(moe_route(&glm, p, MOE_F32, 0, fp, NULL, ip, fp, p, ws1, NULL), MOE_EINVAL, "route T");
  expect(moe_route(&glm, (char*)p + 4, MOE_F32, 1, fp, NULL, ip, fp, p, ws1, NULL), MOE_EINVAL,
         "route misaligned x");
  expect(moe_route(&glm, p, MOE_F32, 1, fp, NULL, ip, fp, p, ws1 - 1, NULL), MOE_ENOSPC,
         "route workspace");
  expect(moe_union(&glm, NULL, 1, ip, ip, ip, ip, NULL), MOE_EINVAL, "union idx");
  expect(moe_union(&glm, ip, 0, ip, ip, ip, ip, NULL), MOE_EINVAL, "union T");
  expect(moe_expert_ffn(&glm, p, p, MOE_F32, NULL, 0, fp, p, ws1, NULL), MOE_EINVAL, "ffn n");
  expect(moe_expert_ffn(&glm, (char*)p + 8, p, MOE_F32, NULL, 1, fp, p, ws1, NULL), MOE_EINVAL,
         "ffn misaligned blob");
  expect(moe_expert_ffn(&glm, p, p, MOE_F32, NULL, 2, fp, p, ws1, NULL), MOE_ENOSPC,
         "ffn workspace");
  expect(moe_layer_forward(&glm, p, MOE_F32, 1, fp, NULL, tab, fp, 16u, 0.f, NULL, p, ws1, NULL),
         MOE_EUNSUPPORTED, "layer flags");

  expect(moe_layer_forward(&glm, p, MOE_BF16, 1, fp, NULL, tab, fp, MOE_RESIDUAL, 0.f, NULL, p,
                           ws1, NULL),
         MOE_EUNSUPPORTED, "layer bf16 residual");
  expect(moe_layer_forward(&glm, p, MOE_F32, 9, fp, NULL, tab, fp, MOE_BATCH_INVARIANT, 0.f, NULL,
                           p, ws1, NULL),
         MOE_EUNSUPPORTED, "layer invariant T = 9");
  expect(moe_layer_forward(&glm, p, MOE_F32, 1, fp, NULL, NULL, fp, 0u, 0.f, NULL, p, ws1, NULL),
         MOE_EINVAL, "layer table");
  expect(moe_layer_forward(&glm, p, MOE_F32, 1, fp, NULL, tab, fp, MOE_PRENORM_RMS, -1.f, NULL, p,
                           ws1, NULL),
         MOE_EINVAL, "layer eps");
  expect(moe_layer_forward(&glm, p, MOE_F32, 2, fp, NULL, tab, fp, 0u, 0.f, NULL, p, ws1, NULL),
         MOE_ENOSPC, "layer workspace");
  expect(moe_layer_forward_cached(&glm, p, MOE_F32, 9, fp, NULL, tab, p, 64, p, fp, 0u, 0.f, NULL,
                                  p, ws1, NULL),
         MOE_EUNSUPPORTED, "cached T = 9");
  expect(moe_layer_forward_cached(&glm, p, MOE_F32, 1, fp, NULL, tab, p, 4, p, fp, 0u, 0.f, NULL,
                                  p, ws1, NULL),
         MOE_EUNSUPPORTED, "cached too few slots");
  expect(moe_layer_forward_noalloc(&glm, p, MOE_F32, 512, fp, NULL, tab, fp, 0u, 0.f, NULL, NULL),
         MOE_ENOSPC, "noalloc past the array");
  expect(moe_layer_forward_noalloc(&glm, p, MOE_F32, 0, fp, NULL, tab, fp, 0u, 0.f, NULL, NULL),
         MOE_EINVAL, "noalloc T = 0");
  expect(moe_layer_forward_noalloc(&bad_d, p, MOE_F32, 1, fp, NULL, tab, fp, 0u, 0.f, NULL, NULL),
         MOE_EUNSUPPORTED, "noalloc dims");
  expect(moe_timing_arm(99, NULL, NULL, 0), MOE_EINVAL, "timing kernel id");
  expect(moe_hbm_read_probe(p, 15, (uint32_t*)p, 1, NULL), MOE_EINVAL, "probe size");
  if (failures) {
    fprintf(stderr, "abi validation: %d failures\n", failures);
    return 1;
  }
  printf("abi validation: all ok\n");
  return 0;
}
