/*
 * A plain C caller of libmoefp8.so written against the eight-operation
 * boundary of the layer's problem statement (routing, permutation, the two
 * FP8 quantisers, the block-scaled grouped GEMM, SwiGLU, the combine and the
 * block transpose), declared HERE by hand rather than taken from
 * include/moefp8.h: if an exported prototype drifts from this boundary (an
 * inserted or reordered parameter), the calls below pass their arguments in
 * the wrong slots and the expected status codes stop matching.
 *
 * Every call fails argument validation on the host (or is an empty
 * problem), so nothing is launched and no GPU is needed.  Prints one line
 * per check; exits 0 when all pass.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

typedef struct ihipStream_t* hipStream_t;
typedef int32_t moe_status;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_ROUTE_SIGMOID_BIAS = 0, MOE_ROUTE_SOFTMAX_GROUPED = 1 } moe_route_mode;
enum { OK = 0, E_NULL = 1, E_SHAPE = 2, E_UNSUP = 3, E_ALIGN = 4, E_WS = 5 };

moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K,
                     int32_t n_groups, int32_t k_per_group, moe_route_mode mode, int32_t normalize_topk,
                     int32_t* topk_idx, float* topk_gate, hipStream_t stream);
moe_status moe_permute_workspace_size(int32_t T, int32_t K, int32_t E, size_t* bytes);
moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E, const uint8_t* xq,
                       const float* xs, int32_t H, int32_t* expert_offsets, int32_t* dst_row,
                       int32_t* src_token, uint8_t* aq, float* as, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
moe_status quant_act_1x128_e4m3(const void* x, moe_dtype x_dtype, int64_t rows, int32_t cols, uint8_t* q,
                                float* scale, hipStream_t stream);
moe_status quant_weight_128x128_e4m3(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows, int32_t cols,
                                     uint8_t* q, float* scale, hipStream_t stream);
moe_status grouped_gemm_fp8_blockscaled(const uint8_t* aq, const float* as, const uint8_t* bq, const float* bs,
                                        const int32_t* group_offsets, int32_t G, int64_t M, int32_t N,
                                        int32_t K, void* c, moe_dtype c_dtype, hipStream_t stream);
moe_status swiglu(const float* gate_up, int64_t M, int32_t I, uint8_t* hq, float* hs, hipStream_t stream);
moe_status moe_combine(const float* y_perm, const int32_t* dst_row, const float* topk_gate,
                       const float* shared, int32_t T, int32_t K, int32_t H, uint16_t* out_bf16,
                       hipStream_t stream);
moe_status fp8_block_transpose(const uint8_t* q, const float* scale, int32_t G, int32_t rows, int32_t cols,
                               uint8_t* qt, float* scale_t, hipStream_t stream);
const char* moe_status_string(moe_status s);
const char* moe_last_error_detail(void);

static int failures = 0;

static void expect(const char* what, moe_status got, moe_status want) {
  const int ok = got == want;
  printf("%s %s: got %d (%s), want %d\n", ok ? "ok  " : "FAIL", what, (int)got, moe_status_string(got),
         (int)want);
  if (!ok) {
    printf("     detail: %s\n", moe_last_error_detail());
    ++failures;
  }
}

int main(void) {
  /* fake device addresses: validation never dereferences them */
  void* P = (void*)(uintptr_t)0x10000;  /* 16-byte aligned */
  void* PM = (void*)(uintptr_t)0x10004; /* 4-byte aligned only */
  hipStream_t S = NULL;
  size_t ws = 0;

  /* routing */
  expect("moe_route E > 1024", moe_route(P, NULL, 4, 2048, 8, 1, 8, MOE_ROUTE_SIGMOID_BIAS, 1, P, P, S), E_UNSUP);
  expect("moe_route K > E", moe_route(P, NULL, 4, 16, 17, 1, 17, MOE_ROUTE_SIGMOID_BIAS, 1, P, P, S), E_SHAPE);
  expect("moe_route G*K' != K", moe_route(P, NULL, 4, 16, 8, 4, 1, MOE_ROUTE_SOFTMAX_GROUPED, 0, P, P, S), E_SHAPE);
  expect("moe_route NULL logits", moe_route(NULL, NULL, 4, 16, 4, 1, 4, MOE_ROUTE_SIGMOID_BIAS, 1, P, P, S), E_NULL);

  /* permutation */
  expect("moe_permute_workspace_size", moe_permute_workspace_size(4096, 8, 256, &ws), OK);
  expect("moe_permute_workspace_size K > E", moe_permute_workspace_size(10, 9, 8, &ws), E_SHAPE);
  expect("moe_permute small workspace", moe_permute(P, 8, 2, 8, NULL, NULL, 0, P, P, P, NULL, NULL, P, 16, S), E_WS);
  expect("moe_permute H % 128", moe_permute(P, 8, 2, 8, P, P, 100, P, P, P, P, P, P, 1 << 20, S), E_SHAPE);
  expect("moe_permute NULL offsets", moe_permute(P, 8, 2, 8, NULL, NULL, 0, NULL, P, P, NULL, NULL, P, 1 << 20, S), E_NULL);

  /* quantisers */
  expect("quant_act cols % 128", quant_act_1x128_e4m3(P, MOE_F32, 4, 100, P, P, S), E_SHAPE);
  expect("quant_act unaligned x", quant_act_1x128_e4m3(PM, MOE_BF16, 4, 128, P, P, S), E_ALIGN);
  expect("quant_act no rows", quant_act_1x128_e4m3(NULL, MOE_F32, 0, 128, NULL, NULL, S), OK);
  expect("quant_weight rows % 128", quant_weight_128x128_e4m3(P, MOE_F32, 2, 100, 128, P, P, S), E_SHAPE);
  expect("quant_weight NULL q", quant_weight_128x128_e4m3(P, MOE_BF16, 2, 128, 128, NULL, P, S), E_NULL);
  expect("quant_weight unaligned q", quant_weight_128x128_e4m3(P, MOE_BF16, 2, 128, 128, PM, P, S), E_ALIGN);
  expect("quant_weight bad dtype", quant_weight_128x128_e4m3(P, (moe_dtype)7, 2, 128, 128, P, P, S), E_UNSUP);

  /* grouped GEMM */
  expect("gemm N % 128", grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, 64, 100, 128, P, MOE_F32, S), E_SHAPE);
  expect("gemm G > 1024", grouped_gemm_fp8_blockscaled(P, P, P, P, P, 2048, 64, 128, 128, P, MOE_F32, S), E_UNSUP);
  expect("gemm NULL offsets", grouped_gemm_fp8_blockscaled(P, P, P, P, NULL, 4, 64, 128, 128, P, MOE_F32, S), E_NULL);
  expect("gemm NULL c", grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, 64, 128, 128, NULL, MOE_BF16, S), E_NULL);
  expect("gemm unaligned bq", grouped_gemm_fp8_blockscaled(P, P, PM, P, P, 4, 64, 128, 128, P, MOE_F32, S), E_ALIGN);
  expect("gemm bad c_dtype", grouped_gemm_fp8_blockscaled(P, P, P, P, P, 4, 64, 128, 128, P, (moe_dtype)5, S), E_UNSUP);
  expect("gemm M = 0", grouped_gemm_fp8_blockscaled(NULL, NULL, NULL, NULL, P, 4, 0, 128, 128, NULL, MOE_F32, S), OK);

  /* SwiGLU, combine, transpose */
  expect("swiglu I % 128", swiglu(P, 4, 100, P, P, S), E_SHAPE);
  expect("swiglu NULL gate_up", swiglu(NULL, 4, 128, P, P, S), E_NULL);
  expect("combine H % 8", moe_combine(P, P, P, NULL, 4, 2, 12, P, S), E_SHAPE);
  expect("combine unaligned shared", moe_combine(P, P, P, PM, 4, 2, 16, P, S), E_ALIGN);
  expect("combine no tokens", moe_combine(NULL, NULL, NULL, NULL, 0, 2, 16, NULL, S), OK);
  expect("transpose rows % 128", fp8_block_transpose(P, P, 2, 100, 128, P, P, S), E_SHAPE);
  expect("transpose NULL qt", fp8_block_transpose(P, P, 2, 128, 128, NULL, P, S), E_NULL);

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "PASSED", failures);
  return failures ? 1 : 0;
}
