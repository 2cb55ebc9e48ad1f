// Token -> expert routing, one 64-lane wavefront per token (the per-token
// work is in route_device.h), and the elementwise binary32 sigmoid.
#include "device_common.h"
#include "host_common.h"
#include "route_device.h"

namespace moefp8 {
namespace {

// sigmoid of every element, the routing's own device function (the same
// binary32 specification), four values per lane.
__global__ __launch_bounds__(256) void sigmoid_kernel(const float* __restrict__ x, int64_t n,
                                                      float* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *reinterpret_cast<const float4*>(x + i);
    *reinterpret_cast<float4*>(y + i) =
        make_float4(spec_sigmoid(v.x), spec_sigmoid(v.y), spec_sigmoid(v.z), spec_sigmoid(v.w));
  } else {
    for (int64_t j = i; j < n; ++j) y[j] = spec_sigmoid(x[j]);
  }
}

template <int PL>
__global__ __launch_bounds__(256) void route_sigmoid_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ bias, int T,
                                                            int E, int K, int normalize,
                                                            int* __restrict__ topk_idx,
                                                            float* __restrict__ topk_gate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together; no barriers below
  route_sigmoid_token<PL>(logits + (int64_t)t * E, bias, E, K, normalize, topk_idx + (int64_t)t * K,
                          topk_gate + (int64_t)t * K);
}

template <int PL>
__global__ __launch_bounds__(256) void route_grouped_kernel(const float* __restrict__ logits, int T,
                                                            int E, int G, int Kp,
                                                            int* __restrict__ topk_idx,
                                                            float* __restrict__ topk_gate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int K = G * Kp;
  route_grouped_token<PL>(logits + (int64_t)t * E, E, G, Kp, topk_idx + (int64_t)t * K,
                          topk_gate + (int64_t)t * K);
}

template <int PL>
struct LaunchRoute {
  static void run(const float* logits, const float* bias, int T, int E, int K, int G, int Kp, int mode,
                  int normalize, int* idx, float* gate, hipStream_t st) {
    const unsigned grid = ceil_div_u(T, 4);
    if (mode == MOE_ROUTE_SIGMOID_BIAS)
      route_sigmoid_kernel<PL><<<grid, 256, 0, st>>>(logits, bias, T, E, K, normalize, idx, gate);
    else
      route_grouped_kernel<PL><<<grid, 256, 0, st>>>(logits, T, E, G, Kp, idx, gate);
  }
};

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E,
                                int32_t K, int32_t n_groups, int32_t k_per_group,
                                moe_route_mode mode, int32_t normalize_topk, int32_t* topk_idx,
                                float* topk_gate, void* stream) {
  clear_detail();
  MOE_REQUIRE(mode == MOE_ROUTE_SIGMOID_BIAS || mode == MOE_ROUTE_SOFTMAX_GROUPED,
              MOE_ERR_UNSUPPORTED, "unknown route mode %d", (int)mode);
  MOE_REQUIRE(T >= 0 && E >= 1, MOE_ERR_SHAPE, "T=%d E=%d", T, E);
  MOE_REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "E=%d > 1024", E);
  MOE_REQUIRE(K >= 1 && K <= E, MOE_ERR_SHAPE, "need 1 <= K <= E (K=%d, E=%d)", K, E);
  if (mode == MOE_ROUTE_SOFTMAX_GROUPED) {
    MOE_REQUIRE(n_groups >= 1 && E % n_groups == 0, MOE_ERR_SHAPE, "E=%d not divisible by n_groups=%d",
                E, n_groups);
    MOE_REQUIRE(k_per_group >= 1 && k_per_group <= E / n_groups, MOE_ERR_SHAPE,
                "need 1 <= k_per_group <= E/n_groups (k_per_group=%d)", k_per_group);
    MOE_REQUIRE(K == n_groups * k_per_group, MOE_ERR_SHAPE, "K=%d != n_groups*k_per_group=%d", K,
                n_groups * k_per_group);
    MOE_REQUIRE(normalize_topk == 0, MOE_ERR_UNSUPPORTED, "grouped softmax gates are not renormalised");
  }
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(logits && topk_idx && topk_gate, MOE_ERR_NULL, "logits, topk_idx and topk_gate are required");
  MOE_REQUIRE(aligned(logits, 4) && aligned(topk_idx, 4) && aligned(topk_gate, 4) && aligned(bias, 4),
              MOE_ERR_ALIGN, "4-byte alignment required");
  hipStream_t st = as_stream(stream);
  const int G = mode == MOE_ROUTE_SOFTMAX_GROUPED ? n_groups : 1;
  const int Kp = mode == MOE_ROUTE_SOFTMAX_GROUPED ? k_per_group : K;
  dispatch_per_lane<LaunchRoute>(E, logits, bias, (int)T, (int)E, (int)K, G, Kp, (int)mode, (int)normalize_topk,
                                 topk_idx, topk_gate, st);
  return after_launch("moe_route", st);
}

extern "C" moe_status moe_sigmoid_f32(const float* x, int64_t n, float* y, void* stream) {
  clear_detail();
  MOE_REQUIRE(n >= 0, MOE_ERR_SHAPE, "n=%lld", (long long)n);
  if (n == 0) return MOE_OK;
  MOE_REQUIRE(x && y, MOE_ERR_NULL, "x and y are required");
  MOE_REQUIRE(aligned(x, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x and y need 16-byte alignment");
  MOE_REQUIRE(n <= kMaxElems, MOE_ERR_UNSUPPORTED, "n=%lld above 2^40", (long long)n);
  const int64_t blocks = (n + 1023) / 1024;
  hipStream_t st = as_stream(stream);
  sigmoid_kernel<<<(unsigned)blocks, 256, 0, st>>>(x, n, y);
  return after_launch("moe_sigmoid_f32", st);
}
