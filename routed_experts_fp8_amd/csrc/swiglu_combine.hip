// Standalone SwiGLU + 1x128 FP8 quantisation, and the gate-weighted combine.
//
// swiglu: h = silu(g) * u per element with the binary32 sigmoid
// specification, then the 1x128 tile quantisation of h (the down-projection
// is an FP8 GEMM too, [DSV3-FP8]).  32 lanes own one 128-wide tile (4 values
// each, float4 loads of g and u), the tile amax is a 32-lane shuffle
// reduction, codes go out as one dword per lane.
//
// combine ([DSV3-MOE], shared + routed experts): out[t] = bf16(sum_k
// gate[t,k] * y_perm[dst_row[t,k]] + shared[t]), summed in slot order in
// binary32 (fixed order, so the result is reproducible).  One workgroup per
// token; each thread carries 4 columns and keeps up to 8 independent 16-byte
// loads in flight (non-temporal: every expert output is read once).
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ gu, int64_t M, int I,
                                                     uint8_t* __restrict__ hq,
                                                     float* __restrict__ hs) {
  const int64_t nvec = M * (int64_t)(I / 4);  // 4 h values per lane
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int qv = I / 4;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v - threadIdx.x % 64 < nvec;
       v += stride) {
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    const bool ok = v < nvec;
    int64_t m = 0;
    int c4 = 0;
    if (ok) {
      m = v / qv;
      c4 = (int)(v % qv);
      const float4 g = *reinterpret_cast<const float4*>(gu + m * 2 * I + 4 * c4);
      const float4 u = *reinterpret_cast<const float4*>(gu + m * 2 * I + I + 4 * c4);
      h[0] = spec_silu(g.x) * u.x;
      h[1] = spec_silu(g.y) * u.y;
      h[2] = spec_silu(g.z) * u.z;
      h[3] = spec_silu(g.w) * u.w;
    }
    float amax = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
    amax = group_max<32>(amax);
    if (ok) {
      const float s = scale_from_amax(amax);
      const uint32_t w = quantize4(Divider(s), h[0], h[1], h[2], h[3]);
      *reinterpret_cast<uint32_t*>(hq + m * I + 4 * c4) = w;
      if ((c4 & 31) == 0) hs[m * (I / 128) + c4 / 32] = s;
    }
  }
}

// Slots are taken 8 at a time: the rows and gates of a batch are
// wave-uniform (scalar loads), the batch's 16-byte loads are all issued
// before the first add, and the adds then run in slot order.  For K <= 8 (one
// batch) the rows and gates are read once per token, outside the column loop.
constexpr int kCombineBatch = 8;

template <bool kOneBatch>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int* __restrict__ dst_row,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ shared, int K,
                                                      int H, uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const float* row[kCombineBatch];
  float g[kCombineBatch];
  auto load_batch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (k0 + j < K) {
        row[j] = y_perm + (int64_t)dst_row[t * K + k0 + j] * H;
        g[j] = gate[t * K + k0 + j];
      }
    }
  };
  if (kOneBatch) load_batch(0);
  for (int c = 4 * threadIdx.x; c < H; c += 4 * blockDim.x) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += kCombineBatch) {
      if (!kOneBatch) load_batch(k0);
      u32x4 y[kCombineBatch];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j)
        if (k0 + j < K) y[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row[j] + c));
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (k0 + j < K) {
          acc[0] = acc[0] + g[j] * __uint_as_float(y[j][0]);
          acc[1] = acc[1] + g[j] * __uint_as_float(y[j][1]);
          acc[2] = acc[2] + g[j] * __uint_as_float(y[j][2]);
          acc[3] = acc[3] + g[j] * __uint_as_float(y[j][3]);
        }
      }
      if (kOneBatch) break;
    }
    if (shared) {
      const u32x4 s4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(shared + t * H + c));
      acc[0] = acc[0] + __uint_as_float(s4[0]);
      acc[1] = acc[1] + __uint_as_float(s4[1]);
      acc[2] = acc[2] + __uint_as_float(s4[2]);
      acc[3] = acc[3] + __uint_as_float(s4[3]);
    }
    uint2 o;
    o.x = bf16_rne_bits(acc[0]) | (bf16_rne_bits(acc[1]) << 16);
    o.y = bf16_rne_bits(acc[2]) | (bf16_rne_bits(acc[3]) << 16);
    *reinterpret_cast<uint2*>(out + t * H + c) = o;
  }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status swiglu(const float* gate_up, int64_t M, int32_t I, uint8_t* hq, float* hs,
                             void* stream) {
  clear_detail();
  MOE_REQUIRE(M >= 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "M=%lld I=%d (I a positive multiple of 128)",
              (long long)M, I);
  MOE_REQUIRE(elems_ok(M, 2 * (int64_t)I), MOE_ERR_UNSUPPORTED, "M=%lld x 2I=%lld above 2^40 elements",
              (long long)M, 2 * (long long)I);
  if (M == 0) return MOE_OK;
  MOE_REQUIRE(gate_up && hq && hs, MOE_ERR_NULL, "gate_up, hq and hs are required");
  MOE_REQUIRE(aligned(gate_up, 16) && aligned(hq, 16) && aligned(hs, 4), MOE_ERR_ALIGN,
              "gate_up and hq need 16-byte alignment");
  hipStream_t st = as_stream(stream);
  const int64_t nvec = M * (I / 4);
  const int64_t need = (nvec + 255) / 256;
  swiglu_kernel<<<(unsigned)(need < 16384 ? need : 16384), 256, 0, st>>>(gate_up, M, I, hq, hs);
  return after_launch("swiglu", st);
}

extern "C" moe_status moe_combine(const float* y_perm, const int32_t* dst_row,
                                  const float* topk_gate, const float* shared, int32_t T,
                                  int32_t K, int32_t H, uint16_t* out_bf16, void* stream) {
  clear_detail();
  MOE_REQUIRE(T >= 0 && K >= 1 && H > 0 && H % 8 == 0, MOE_ERR_SHAPE, "T=%d K=%d H=%d (H must be a positive multiple of 8)", T, K, H);
  MOE_REQUIRE(elems_ok((int64_t)T * K, H), MOE_ERR_UNSUPPORTED, "T*K=%lld x H=%d above 2^40 elements",
              (long long)T * K, H);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y_perm && dst_row && topk_gate && out_bf16, MOE_ERR_NULL,
              "y_perm, dst_row, topk_gate and out_bf16 are required");
  MOE_REQUIRE(aligned(y_perm, 16) && aligned(out_bf16, 16) && aligned(shared, 16) &&
                  aligned(dst_row, 4) && aligned(topk_gate, 4),
              MOE_ERR_ALIGN, "y_perm, shared and out need 16-byte alignment");
  hipStream_t st = as_stream(stream);
  if (K <= kCombineBatch)
    combine_kernel<true><<<(unsigned)T, 256, 0, st>>>(y_perm, dst_row, topk_gate, shared, K, H, out_bf16);
  else
    combine_kernel<false><<<(unsigned)T, 256, 0, st>>>(y_perm, dst_row, topk_gate, shared, K, H, out_bf16);
  return after_launch("moe_combine", st);
}
