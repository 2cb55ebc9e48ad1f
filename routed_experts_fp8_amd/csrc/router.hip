// Router projection and the aux-loss-free balancing bias update
// ([DSV3-MOE]: sigmoid affinity scores from the router, and a per-expert
// bias adjusted to balance the load, in place of an auxiliary loss).
//
// router_kernel: logits[t, e] = sum_h x[t, h] * W_r[e, h] with x bf16 and
//   W_r float32 [E, H] (the gating path stays in float32, unlike the FP8
//   expert GEMMs), float32 products and sums on the matrix cores
//   (V_MFMA_F32_16X16X4_F32).  One workgroup per 64 (or, when that gives
//   too few workgroups, 32) tokens x 64 experts, 4 waves of 32 (16) x 32;
//   the reduction over H runs in chunks of 64 columns
//   staged through LDS as float32 (x widened on the way), the next chunk's
//   global loads in flight during this chunk's products.  At the
//   DeepSeek-V3 shape (4096 x 256 x 7168, 15 GFLOP) it is bound by the
//   float32 matrix rate.
//
// bias_update_kernel: b_e <- b_e - gamma * sign(load_e - mean) from one
//   step's per-expert grouped-row counts, the comparison with the mean taken
//   exactly on integers (load_e * E against the total), one binary32
//   subtraction of +-gamma or 0.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

template <int TT>  // tokens per workgroup tile: 64 or 32
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                     int T, int H, int E, float* __restrict__ logits) {
  constexpr int NI = TT / 32;  // 16-token instruction tiles per wave
  __shared__ __attribute__((aligned(16))) float sX[TT][68];  // tokens x 64 columns (+4 against bank conflicts)
  __shared__ __attribute__((aligned(16))) float sW[64][68];  // experts x 64 columns
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * (TT / 2), wn = (wave & 1) * 32;
  // loaders: x row rx, 64 / (256 / TT) bf16 columns from cx; W row rw, 16 columns from cw
  constexpr int XPT = 64 * TT / 256;  // bf16 per thread: 16 or 8
  const int rx = tid / (64 / XPT), cx = (tid % (64 / XPT)) * XPT;
  const int rw = tid >> 2, cw = (tid & 3) * 16;
  const bool xr = t0 + rx < T, wr = e0 + rw < E;
  const uint16_t* xp = x + (int64_t)(xr ? t0 + rx : 0) * H + cx;
  const float* wp = w + (int64_t)(wr ? e0 + rw : 0) * H + cw;

  uint4 xa, xb;
  float4 w0, w1, w2, w3;
  auto fetch = [&](int h0) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    const float4 zf = make_float4(0.f, 0.f, 0.f, 0.f);
    xa = xr ? *reinterpret_cast<const uint4*>(xp + h0) : z;
    xb = (XPT == 16 && xr) ? *reinterpret_cast<const uint4*>(xp + h0 + 8) : z;
    w0 = wr ? *reinterpret_cast<const float4*>(wp + h0) : zf;
    w1 = wr ? *reinterpret_cast<const float4*>(wp + h0 + 4) : zf;
    w2 = wr ? *reinterpret_cast<const float4*>(wp + h0 + 8) : zf;
    w3 = wr ? *reinterpret_cast<const float4*>(wp + h0 + 12) : zf;
  };

  v4f acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  for (int h0 = 0; h0 < H; h0 += 64) {
    __syncthreads();  // every wave is done with the previous chunk
    {
      float4* dx = reinterpret_cast<float4*>(&sX[rx][cx]);
      const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int i = 0; i < XPT / 4; ++i)
        dx[i] = make_float4(__uint_as_float(xw[2 * i] << 16), __uint_as_float(xw[2 * i] & 0xffff0000u),
                            __uint_as_float(xw[2 * i + 1] << 16), __uint_as_float(xw[2 * i + 1] & 0xffff0000u));
      float4* dw = reinterpret_cast<float4*>(&sW[rw][cw]);
      dw[0] = w0, dw[1] = w1, dw[2] = w2, dw[3] = w3;
    }
    __syncthreads();
    if (h0 + 64 < H) fetch(h0 + 64);
#pragma unroll
    for (int k = 0; k < 64; k += 4) {
      float a[NI], b[2];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = sX[wm + 16 * i + (lane & 15)][k + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sW[wn + 16 * j + (lane & 15)][k + (lane >> 4)];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // lane holds tokens wm + 16 i + 4 (lane / 16) + v of expert wn + 16 j + lane % 16
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn + 16 * j + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + wm + 16 * i + 4 * (lane >> 4) + v;
        if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i][j][v];
      }
    }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int* __restrict__ off, int E, float gamma,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)off[e + 1] - off[e];
  const int64_t total = (int64_t)off[E] - off[0];
  const int64_t d = load * E - total;  // sign of load - total / E, exactly
  const float step = d > 0 ? gamma : (d < 0 ? -gamma : 0.0f);
  bias[e] = bias[e] - step;
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_router_logits(const uint16_t* x_bf16, const float* w_router, int32_t T, int32_t H,
                                        int32_t E, float* logits, void* stream) {
  clear_detail();
  MOE_REQUIRE(T >= 0 && E >= 1 && H > 0 && H % 64 == 0, MOE_ERR_SHAPE,
              "T=%d H=%d E=%d (H a positive multiple of 64, E >= 1)", T, H, E);
  MOE_REQUIRE(((int64_t)E + 63) / 64 <= 65535, MOE_ERR_UNSUPPORTED, "E=%d too large", E);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x_bf16 && w_router && logits, MOE_ERR_NULL, "x, w_router and logits are required");
  MOE_REQUIRE(aligned(x_bf16, 16) && aligned(w_router, 16) && aligned(logits, 4), MOE_ERR_ALIGN,
              "x and w_router need 16-byte alignment");
  hipStream_t s = as_stream(stream);
  // 32-token tiles when 64-token ones would leave compute units without a
  // second workgroup
  const unsigned ge = (unsigned)(((int64_t)E + 63) / 64);
  if (((int64_t)T + 63) / 64 * ge < 512)
    router_kernel<32><<<dim3((unsigned)((T + 31) / 32), ge), 256, 0, s>>>(x_bf16, w_router, T, H, E, logits);
  else
    router_kernel<64><<<dim3((unsigned)(((int64_t)T + 63) / 64), ge), 256, 0, s>>>(x_bf16, w_router, T, H, E, logits);
  return after_launch("moe_router_logits", s);
}

extern "C" moe_status moe_bias_update(const int32_t* expert_offsets, int32_t E, float gamma, float* bias,
                                      void* stream) {
  clear_detail();
  MOE_REQUIRE(E >= 1, MOE_ERR_SHAPE, "E=%d", E);
  MOE_REQUIRE(expert_offsets && bias, MOE_ERR_NULL, "expert_offsets and bias are required");
  MOE_REQUIRE(aligned(expert_offsets, 4) && aligned(bias, 4), MOE_ERR_ALIGN, "4-byte alignment required");
  hipStream_t s = as_stream(stream);
  bias_update_kernel<<<(unsigned)((E + 255) / 256), 256, 0, s>>>(expert_offsets, E, gamma, bias);
  return after_launch("moe_bias_update", s);
}
