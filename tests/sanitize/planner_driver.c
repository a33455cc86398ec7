/* planner_driver.c -- host-sanitizer driver (tests/test_host_sanitizers.py) for
 * the library's planner and argument validation, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer: dg_select_config over a grid of kinds and
 * shapes (with the plan's invariants checked), and every entry point's
 * rejection of bad arguments, which happens before any HIP call. */
#include <stdint.h>
#include <stdio.h>

#include "dg.h"

static int bad = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);     \
      bad++;                                                            \
    }                                                                   \
  } while (0)

int main(void) {
  const int ms[] = {1, 17, 64, 127, 128, 129, 256, 300, 4096, 65536};
  const int ns[] = {1, 16, 130, 2112, 4096, 7168, 24576, 32768};
  const int ks[] = {128, 512, 2048, 4608, 7168, 16384, 1 << 20};
  const int gs[] = {1, 2, 4, 16, 256};
  long plans = 0;
  for (int kind = 0; kind <= 11; ++kind)
    for (unsigned a = 0; a < sizeof(ms) / sizeof(ms[0]); ++a)
      for (unsigned b = 0; b < sizeof(ns) / sizeof(ns[0]); ++b)
        for (unsigned c = 0; c < sizeof(ks) / sizeof(ks[0]); ++c)
          for (unsigned d = 0; d < sizeof(gs) / sizeof(gs[0]); ++d)
            for (int cus = 1; cus <= 256; cus *= 16) {
              dg_tile_config cfg;
              const dg_status s = dg_select_config(kind, ms[a], ns[b], ks[c], gs[d], cus, &cfg);
              if (s != DG_SUCCESS) continue;
              ++plans;
              const int bf16 = kind == DG_KIND_BF16 || kind == DG_KIND_CONTIGUOUS_BF16 || kind == DG_KIND_MASKED_BF16;
              const int kblocks = (bf16 ? 2 * ks[c] : ks[c]) / 128;
              CHECK(cfg.block_m > 0 && cfg.block_n > 0 && cfg.block_n % 16 == 0);
              CHECK(cfg.waves_m > 0 && cfg.waves_n > 0);
              CHECK(cfg.tiles >= 1 && cfg.grid >= 1);
              CHECK(cfg.k_splits >= 1 && cfg.k_splits <= kblocks);
              CHECK((long)cfg.grid <= ((long)cfg.tiles * cfg.k_splits + 7) / 8 * 8);
              CHECK(cfg.grid <= 8 || cfg.grid % 8 == 0);
            }
  CHECK(plans > 1000);
  /* rejected queries */
  dg_tile_config cfg;
  CHECK(dg_select_config(12, 128, 128, 128, 1, 256, &cfg) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_select_config(7, 128, 384, 128, 1, 256, &cfg) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_select_config(0, 0, 128, 128, 1, 256, &cfg) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_select_config(0, 128, 128, 128, 1, 256, NULL) == DG_ERROR_INVALID_VALUE);
  /* argument validation, before any HIP call (fake, never dereferenced addresses) */
  void* p = (void*)(uintptr_t)0x10000;
  void* mis = (void*)(uintptr_t)0x10001;
  const float* f = (const float*)p;
  CHECK(dg_gemm_fp8_nt(NULL, f, p, f, p, 1, 1, 128, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_gemm_fp8_nt(p, f, p, f, p, 1, 1, 100, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_gemm_fp8_nt(mis, f, p, f, p, 1, 1, 128, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_gemm_fp8_nt_ue8m0(p, f, p, f, p, -1, 1, 128, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_gemm_bf16_nt(p, p, p, 1, 1, 100, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_bf16_contiguous(p, p, p, NULL, 128, 8, 128, 2, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_grouped_bf16_masked(p, p, p, (const int32_t*)p, 2, 256, 8, 100, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_fp8_contiguous(p, f, p, f, p, (const int32_t*)p, 100, 8, 128, 2, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_fp8_contiguous(p, f, p, f, p, NULL, 128, 8, 128, 2, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_grouped_fp8_contiguous_swiglu(p, f, p, f, p, (float*)p, (const int32_t*)p, 128, 384, 128, 2, NULL) ==
        DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_fp8_contiguous_swiglu(p, f, p, f, p, NULL, (const int32_t*)p, 128, 512, 128, 2, NULL) ==
        DG_ERROR_INVALID_VALUE);
  CHECK(dg_grouped_fp8_masked(p, f, p, f, p, (const int32_t*)p, 0, 256, 8, 128, NULL) == DG_ERROR_INVALID_VALUE);
  const int32_t* w = (const int32_t*)p;
  CHECK(dg_gemm_fp8_nt_ue8m0_packed(p, w, p, w, p, 1, 1, 100, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_fp8_contiguous_ue8m0_packed(p, w, p, w, p, NULL, 128, 8, 128, 2, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_grouped_fp8_masked_ue8m0_packed(p, w, p, w, p, w, 2, 256, 8, 200, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_grouped_fp8_masked_noalloc(p, f, p, f, p, NULL, 2, 256, 8, 128, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_grouped_fp8_masked_noalloc(p, f, p, f, p, (const int32_t*)p, 2, 256, 8, 200, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_wgrad_fp8_nt(p, f, p, f, (float*)p, 8, 8, 0, NULL) == DG_ERROR_INVALID_VALUE);
  const int32_t ks_bad[3] = {128, -128, 0}, ks_odd[2] = {128, 100};
  CHECK(dg_k_grouped_wgrad_fp8_nt(p, f, p, f, (float*)p, ks_bad, 3, 8, 8, NULL) == DG_ERROR_INVALID_VALUE);
  CHECK(dg_k_grouped_wgrad_fp8_nt(p, f, p, f, (float*)p, ks_odd, 2, 8, 8, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_k_grouped_wgrad_fp8_nt(p, f, p, f, (float*)p, ks_bad, 300, 8, 8, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_quantize_fp8_1x128((const float*)p, p, (float*)p, 4, 100, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_quantize_fp8_1x128_transposed((const float*)p, p, (float*)p, 100, 8, NULL) == DG_ERROR_UNSUPPORTED);
  CHECK(dg_swiglu_quantize_fp8_1x128(p, p, (float*)p, 4, 100, NULL) == DG_ERROR_UNSUPPORTED);
  for (int s = 0; s <= 4; ++s) CHECK(dg_status_string((dg_status)s) != NULL);
  printf("plans=%ld bad=%d\n", plans, bad);
  return bad != 0;
}
