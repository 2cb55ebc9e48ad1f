// Token -> expert routing, one 64-lane wavefront per token.
//
// SIGMOID_BIAS ([DSV3-MOE]): sigmoid affinity per expert, a per-expert bias
// shifts the selection key, the K best keys win (lower expert index on equal
// keys), gates are the unbiased sigmoid scores, optionally normalised over
// the K winners in slot order.
// SOFTMAX_GROUPED ([PANGU-MOGE]): experts in G equal groups, each group keeps
// its K' largest logits (equivalently its K' largest softmax scores), gates
// are the global softmax scores (float64 on the device, rounded once to
// float32), unselected experts score 0.
//
// Each lane keeps the keys of experts e = lane + 64*i in registers
// (E <= 1024 -> at most 16 per lane).  Every pick is a wave-wide arg-max on
// (key, -index) by butterfly shuffles, so K picks cost K reductions and no
// memory traffic beyond the logits row.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

constexpr int kMaxPerLane = 16;  // E <= 1024

struct Cand {
  float key;
  int e;      // expert index, INT_MAX when empty
  float val;  // value carried to the winner (sigmoid score / logit)
};

__device__ __forceinline__ bool better(float k1, int e1, float k2, int e2) {
  return k1 > k2 || (k1 == k2 && e1 < e2);
}

__device__ __forceinline__ Cand wave_argmax(Cand c) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float k2 = __shfl_xor(c.key, m, 64);
    const int e2 = __shfl_xor(c.e, m, 64);
    const float v2 = __shfl_xor(c.val, m, 64);
    if (better(k2, e2, c.key, c.e)) {
      c.key = k2;
      c.e = e2;
      c.val = v2;
    }
  }
  return c;
}

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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave exits together; no barriers below
  const float* row = logits + (int64_t)t * E;
  float key[PL], sc[PL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    sc[i] = 0.0f;
    key[i] = -INFINITY;
    if (e < E) {
      sc[i] = spec_sigmoid(row[e]);
      key[i] = sc[i] + (bias ? bias[e] : 0.0f);
    } else {
      taken |= 1u << i;
    }
  }
  // slot k's expert and score are kept by lane k % 64 in register k / 64
  int slot_e[PL];
  float slot_s[PL];
  float total = 0.0f;
  for (int k = 0; k < K; ++k) {
    Cand c{-INFINITY, 0x7fffffff, 0.0f};
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (!(taken >> i & 1u) && better(key[i], e, c.key, c.e)) {
        c.key = key[i];
        c.e = e;
        c.val = sc[i];
      }
    }
    c = wave_argmax(c);
    if ((c.e & 63) == lane) taken |= 1u << (c.e >> 6);
    total = total + c.val;  // slot order, binary32 (identical in every lane)
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      if ((k >> 6) == i && (k & 63) == lane) {
        slot_e[i] = c.e;
        slot_s[i] = c.val;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int k = lane + 64 * i;
    if (k < K) {
      topk_idx[(int64_t)t * K + k] = slot_e[i];
      topk_gate[(int64_t)t * K + k] = normalize ? slot_s[i] / total : slot_s[i];
    }
  }
}

template <int PL>
__global__ __launch_bounds__(256) void route_grouped_kernel(const float* __restrict__ logits, int T,
                                                            int E, int G, int Kp,
                                                            int* __restrict__ topk_idx,
                                                            float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  const int per = E / G, K = G * Kp;
  float l[PL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    l[i] = e < E ? row[e] : -INFINITY;
    mx = fmaxf(mx, l[i]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  double z[PL];
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    z[i] = e < E ? exp((double)l[i] - (double)mx) : 0.0;
    sum += z[i];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
  uint32_t taken = 0;
  for (int g = 0; g < G; ++g) {
    const int lo = g * per, hi = lo + per;
    for (int kk = 0; kk < Kp; ++kk) {
      Cand c{-INFINITY, 0x7fffffff, 0.0f};
      double zc = 0.0;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        if (e >= lo && e < hi && !(taken >> i & 1u) && better(l[i], e, c.key, c.e)) {
          c.key = l[i];
          c.e = e;
          zc = z[i];
        }
      }
      // carry z through the reduction as two 32-bit halves
      int zlo = __double2loint(zc), zhi = __double2hiint(zc);
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float k2 = __shfl_xor(c.key, m, 64);
        const int e2 = __shfl_xor(c.e, m, 64);
        const int lo2 = __shfl_xor(zlo, m, 64), hi2 = __shfl_xor(zhi, m, 64);
        if (better(k2, e2, c.key, c.e)) {
          c.key = k2;
          c.e = e2;
          zlo = lo2;
          zhi = hi2;
        }
      }
      if ((c.e & 63) == lane) taken |= 1u << (c.e >> 6);
      if (lane == 0) {
        const int k = g * Kp + kk;
        topk_idx[(int64_t)t * K + k] = c.e;
        topk_gate[(int64_t)t * K + k] = (float)(__hiloint2double(zhi, zlo) / sum);
      }
    }
  }
}

template <int PL>
void launch_route(const float* logits, const float* bias, int T, int E, int K, int G, int Kp,
                  int mode, int normalize, int* idx, float* gate, hipStream_t st) {
  const unsigned grid = ceil_div_u(T, 4);
  if (mode == MOE_ROUTE_SIGMOID_BIAS)
    route_sigmoid_kernel<PL><<<grid, 256, 0, st>>>(logits, bias, T, E, K, normalize, idx, gate);
  else
    route_grouped_kernel<PL><<<grid, 256, 0, st>>>(logits, T, E, G, Kp, idx, gate);
}

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
  const int pl = (E + 63) / 64;
  const int G = mode == MOE_ROUTE_SOFTMAX_GROUPED ? n_groups : 1;
  const int Kp = mode == MOE_ROUTE_SOFTMAX_GROUPED ? k_per_group : K;
  if (pl <= 1)
    launch_route<1>(logits, bias, T, E, K, G, Kp, mode, normalize_topk, topk_idx, topk_gate, st);
  else if (pl <= 2)
    launch_route<2>(logits, bias, T, E, K, G, Kp, mode, normalize_topk, topk_idx, topk_gate, st);
  else if (pl <= 4)
    launch_route<4>(logits, bias, T, E, K, G, Kp, mode, normalize_topk, topk_idx, topk_gate, st);
  else if (pl <= 8)
    launch_route<8>(logits, bias, T, E, K, G, Kp, mode, normalize_topk, topk_idx, topk_gate, st);
  else
    launch_route<kMaxPerLane>(logits, bias, T, E, K, G, Kp, mode, normalize_topk, topk_idx,
                              topk_gate, st);
  return after_launch("moe_route", st);
}

extern "C" moe_status moe_sigmoid_f32(const float* x, int64_t n, float* y, void* stream) {
  clear_detail();
  MOE_REQUIRE(n >= 0, MOE_ERR_SHAPE, "n=%lld", (long long)n);
  if (n == 0) return MOE_OK;
  MOE_REQUIRE(x && y, MOE_ERR_NULL, "x and y are required");
  MOE_REQUIRE(aligned(x, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x and y need 16-byte alignment");
  const int64_t blocks = (n + 1023) / 1024;
  MOE_REQUIRE(blocks < (1LL << 31), MOE_ERR_UNSUPPORTED, "n=%lld too large", (long long)n);
  hipStream_t st = as_stream(stream);
  sigmoid_kernel<<<(unsigned)blocks, 256, 0, st>>>(x, n, y);
  return after_launch("moe_sigmoid_f32", st);
}
