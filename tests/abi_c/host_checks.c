/*
 * Host-side argument checks of every libmoefp8 entry point, driven from C
 * against include/moefp8.h, for a build of the library whose host code runs
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  Besides the usual
 * bad arguments (NULLs, misalignment, sizes off the 128 grid) the calls use
 * extreme sizes (INT32_MAX tokens, 2^40 rows, ...) so that any size product
 * a check computes in too narrow a type overflows visibly.
 *
 * Every call fails validation or is an empty problem that launches nothing,
 * so no GPU is needed.  Prints one line per failed check; exits 0 when all
 * pass.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moefp8.h"

static int failures = 0, checks = 0;

#define CHECK(call, want)                                                                      \
  do {                                                                                         \
    const moe_status got_ = (call);                                                            \
    ++checks;                                                                                  \
    if (got_ != (want)) {                                                                      \
      ++failures;                                                                              \
      printf("FAIL line %d: %s -> %d (%s), want %d\n", __LINE__, #call, got_,                  \
             moe_last_error_detail(), (want));                                                 \
    }                                                                                          \
  } while (0)

enum { OK = MOE_OK, NUL = MOE_ERR_NULL, SHP = MOE_ERR_SHAPE, UNS = MOE_ERR_UNSUPPORTED, ALI = MOE_ERR_ALIGN,
       WSP = MOE_ERR_WORKSPACE };

int main(void) {
  /* fake device pointers: never dereferenced, only checked for NULL/alignment */
  void* P = (void*)(uintptr_t)0x10000;
  void* PM = (void*)(uintptr_t)0x10004; /* 4-byte, not 16-byte aligned */
  void* P2 = (void*)(uintptr_t)0x10002; /* 2-byte aligned */
  void* S = NULL;
  const int32_t IMAX = INT32_MAX;
  const int64_t BIG = (int64_t)1 << 40;
  size_t sz = 0;
  int64_t rows = 0;
  const moe_route_mode SIG = MOE_ROUTE_SIGMOID_BIAS, GRP = MOE_ROUTE_SOFTMAX_GROUPED;

  for (int s = -2; s < 10; ++s) {
    const char* t = moe_status_string(s);
    ++checks;
    if (!t || !*t) {
      ++failures;
      printf("FAIL status string %d\n", s);
    }
  }

  /* routing */
  CHECK(moe_route(P, NULL, 4, 2048, 8, 1, 8, SIG, 1, P, P, S), UNS);
  CHECK(moe_route(P, NULL, 4, 16, 17, 1, 17, SIG, 1, P, P, S), SHP);
  CHECK(moe_route(P, NULL, -1, 16, 4, 1, 4, SIG, 1, P, P, S), SHP);
  CHECK(moe_route(P, NULL, 4, 18, 4, 4, 1, GRP, 0, P, P, S), SHP);
  CHECK(moe_route(P, NULL, 4, 16, 4, 4, 1, GRP, 1, P, P, S), UNS);
  CHECK(moe_route(NULL, NULL, IMAX, 1024, 1024, 1, 1024, SIG, 1, P, P, S), NUL);
  CHECK(moe_route(P, NULL, 0, 16, 4, 1, 4, SIG, 1, NULL, NULL, S), OK);
  CHECK(moe_route(P, NULL, 4, 16, 4, 1, 4, (moe_route_mode)9, 1, P, P, S), UNS);
  CHECK(moe_sigmoid_f32(P, -1, P, S), SHP);
  CHECK(moe_sigmoid_f32(P, INT64_MAX, P, S), UNS);
  CHECK(moe_sigmoid_f32(PM, 16, P, S), ALI);
  CHECK(moe_sigmoid_f32(NULL, 0, NULL, S), OK);

  /* permutation */
  CHECK(moe_permute_workspace_size(IMAX, 1024, 1024, &sz), OK);
  CHECK(moe_permute_workspace_size(10, 9, 8, &sz), SHP);
  CHECK(moe_permute_workspace_size(10, 8, 2048, &sz), UNS);
  CHECK(moe_permute(P, IMAX, 1024, 1024, NULL, NULL, 0, P, P, P, NULL, NULL, P, SIZE_MAX, S), UNS); /* T*K */
  CHECK(moe_permute(P, 8, 2, 8, P, NULL, 128, P, P, P, P, P, P, 1 << 20, S), NUL);
  CHECK(moe_permute(P, 8, 2, 8, P, P, 100, P, P, P, P, P, P, 1 << 20, S), SHP);
  CHECK(moe_permute(P, 8, 2, 8, PM, P, 128, P, P, P, P, P, P, 1 << 20, S), ALI);
  CHECK(moe_permute(P, 8, 2, 8, NULL, NULL, 0, P, P, P, NULL, NULL, P, 16, S), WSP);
  CHECK(moe_permute_noalloc(P, 600000, 2, 256, NULL, NULL, 0, P, P, P, NULL, NULL, S), WSP);
  CHECK(moe_permute_noalloc(P, IMAX, 1024, 1024, NULL, NULL, 0, P, P, P, NULL, NULL, S), UNS);
  CHECK(moe_route_permute_workspace_size(IMAX, 1024, 1024, &sz), OK);
  CHECK(moe_route_permute(P, NULL, IMAX, 1024, 1024, 1, 1024, SIG, 1, P, P, P, P, P, P, SIZE_MAX, S), UNS);
  CHECK(moe_route_permute(P, NULL, 4, 16, 4, 1, 4, SIG, 1, P, P, P, P, P, PM, 1 << 20, S), ALI);
  CHECK(moe_route_permute(P, NULL, 4, 16, 4, 1, 4, SIG, 1, P, P, P, P, P, P, 255, S), WSP);

  /* quantisers and transpose */
  CHECK(quant_act_1x128_e4m3(P, MOE_F32, BIG, 128, P, P, S), UNS);
  CHECK(quant_act_1x128_e4m3(P, MOE_F32, 4, 100, P, P, S), SHP);
  CHECK(quant_act_1x128_e4m3(P, MOE_F32, -1, 128, P, P, S), SHP);
  CHECK(quant_act_1x128_e4m3(NULL, MOE_F32, 0, 128, NULL, NULL, S), OK);
  CHECK(quant_weight_128x128_e4m3(P, MOE_BF16, IMAX, 1 << 30, 1 << 30, P, P, S), UNS);
  CHECK(quant_weight_128x128_e4m3(P, MOE_BF16, 2, 100, 128, P, P, S), SHP);
  CHECK(quant_weight_128x128_e4m3_t(P, MOE_BF16, 2, 128, 128, P, P, P, NULL, S), NUL);
  CHECK(quant_weight_128x128_e4m3_t(P, MOE_BF16, IMAX, 1 << 30, 1 << 30, P, P, P, P, S), UNS);
  CHECK(fp8_block_transpose(P, P, 2, 100, 128, P, P, S), SHP);
  CHECK(fp8_block_transpose(P, P, IMAX, 1 << 30, 1 << 30, P, P, S), UNS);
  CHECK(fp8_block_transpose(NULL, NULL, 0, 128, 128, NULL, NULL, S), OK);

  /* grouped GEMMs */
  CHECK(grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, 64, 100, 128, P, MOE_F32, S), SHP);
  CHECK(grouped_gemm_fp8_blockscaled(P, P, P, P, P, 2048, 64, 128, 128, P, MOE_F32, S), UNS);
  CHECK(grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, BIG, 128, 128, P, MOE_F32, S), UNS);
  CHECK(grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, 64, 128, IMAX - 127, P, MOE_F32, S), UNS);
  CHECK(grouped_gemm_fp8_blockscaled(P, P, P, P, P, 1024, (int64_t)IMAX - 1, 1 << 30, 128, P, MOE_F32, S), UNS);
  CHECK(grouped_gemm_fp8_blockscaled(PM, P, P, P, P, 4, 64, 128, 128, P, MOE_F32, S), ALI);
  CHECK(grouped_gemm_fp8_blockscaled(NULL, NULL, NULL, NULL, P, 4, 0, 128, 128, NULL, MOE_F32, S), OK);
  CHECK(grouped_gemm_fp8_blockscaled_gather(P, P, P, BIG, P, P, P, 4, 64, 128, 128, P, MOE_F32, S), UNS);
  CHECK(grouped_gemm_fp8_blockscaled_gather(P, P, NULL, 16, P, P, P, 4, 64, 128, 128, P, MOE_F32, S), NUL);
  CHECK(grouped_gemm_fp8_swiglu(P, P, NULL, 0, P, P, P, 4, 64, 100, 128, P, P, S), SHP);
  CHECK(grouped_gemm_fp8_swiglu(P, P, NULL, 0, P, P, P, 4, 64, 1 << 30, 128, P, P, S), UNS);
  CHECK(grouped_gemm_fp8_combine_workspace_size(IMAX, IMAX - 127, &sz), OK);
  CHECK(grouped_gemm_fp8_combine(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, NULL, 16, 3, P, P, 1 << 20, S), SHP);
  CHECK(grouped_gemm_fp8_combine(P, P, P, P, P, 4, (int64_t)IMAX * 4, 256, 128, P, P, P, P, NULL, IMAX, 4, P, P,
                                 SIZE_MAX, S), UNS);
  CHECK(grouped_gemm_fp8_combine(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, NULL, 16, 4, P, P, 63, S), WSP);

  /* SwiGLU and combine */
  CHECK(swiglu(P, BIG, 1 << 30, P, P, S), UNS);
  CHECK(swiglu(P, 4, 100, P, P, S), SHP);
  CHECK(moe_combine(P, P, P, NULL, 4, 2, 12, P, S), SHP);
  CHECK(moe_combine(P, P, P, PM, 4, 2, 16, P, S), ALI);
  CHECK(moe_combine(NULL, NULL, NULL, NULL, 0, 2, 16, NULL, S), OK);

  /* backward */
  CHECK(moe_combine_backward(P, P, P, P, 4, 2, 100, P, P, P, NULL, S), SHP);
  CHECK(moe_combine_backward(P, P, P, P, IMAX, 16, 1 << 30, P, P, P, NULL, S), UNS);
  CHECK(moe_combine_backward(P, P, P, P, 4, 2, 128, P, P, P, P2, S), ALI);
  CHECK(swiglu_backward(P, P, BIG, 1 << 30, P, P, NULL, S), UNS);
  CHECK(swiglu_backward(P, P, 4, 128, P, P, PM, S), ALI);
  CHECK(moe_route_backward(P, P, P, 4, 128, 65, SIG, 1, P, S), UNS);
  CHECK(moe_route_backward(P, P, P, IMAX, 1024, 64, SIG, 1, NULL, S), NUL);
  CHECK(moe_route_backward(NULL, NULL, NULL, 0, 8, 2, GRP, 0, NULL, S), OK);

  /* weight gradients */
  CHECK(moe_wgrad_padded_rows(INT64_MAX, 1024, &rows), UNS);
  CHECK(moe_wgrad_padded_rows(-1, 1, &rows), SHP);
  CHECK(moe_wgrad_padded_rows(300, 4, &rows), OK);
  CHECK(quant_act_128x1_grouped_e4m3(P, MOE_F32, 0, 300, 100, NULL, NULL, P, 4, 300, 896, P, P, P, S), SHP);
  CHECK(quant_act_128x1_grouped_e4m3(P, MOE_F32, 0, BIG, 1 << 30, NULL, NULL, P, 1024, BIG, INT64_MAX & ~(int64_t)127,
                                     P, P, P, S),
        UNS);
  CHECK(grouped_wgrad_fp8(P, P, P, P, P, 4, 128, 128, 200, P, MOE_F32, 0, S), SHP);
  CHECK(grouped_wgrad_fp8(P, P, P, P, P, 1024, 1 << 30, 1 << 30, 256, P, MOE_F32, 0, S), UNS);
  CHECK(grouped_wgrad_fp8(P, P, P, P, P, 4, 128, 128, ((int64_t)1 << 29) + 128, P, MOE_F32, 0, S), UNS);
  CHECK(grouped_wgrad_fp8(P, P, P, P, P, 4, 128, 128, 256, (void*)(uintptr_t)0x10008, MOE_F32, 0, S), ALI);

  /* router */
  CHECK(moe_router_logits(P, P, 4, 100, 8, P, S), SHP);
  CHECK(moe_router_logits(P, P, IMAX, 1 << 30, IMAX, P, S), UNS);
  CHECK(moe_router_logits(NULL, NULL, 0, 128, 8, NULL, S), OK);
  CHECK(moe_bias_update(P, 0, 0.1f, P, S), SHP);
  CHECK(moe_bias_update(P, 8, 0.1f, P2, S), ALI);

  /* measurement helper */
  {
    double fl = 0.0;
    CHECK(moe_probe_mfma_fp8(0x38, 10, 0, 8, P, &fl, S), SHP);
    CHECK(moe_probe_mfma_fp8(0x38, -1, 1, 8, P, &fl, S), SHP);
    CHECK(moe_probe_mfma_fp8(0x38, INT64_MAX, 1, 8, P, &fl, S), SHP);
    CHECK(moe_probe_mfma_fp8(0x38, 10, 1, 17, P, &fl, S), SHP);
    CHECK(moe_probe_mfma_fp8(0x38, 10, 1, 8, NULL, &fl, S), NUL);
    CHECK(moe_probe_mfma_fp8(0x38, 10, 1, 8, P, NULL, S), NUL);
    CHECK(moe_probe_mfma_fp8(0x38, 10, 1, 8, P2, &fl, S), ALI);
  }

  printf("%d checks, %d failed\n%s\n", checks, failures, failures ? "FAILED" : "PASSED");
  return failures ? 1 : 0;
}
