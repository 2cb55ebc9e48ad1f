// Input-side backward of the routed-expert layer ([KANANA-FP8]: the
// backward expert GEMMs run in FP8 on the block-transposed forward weights;
// [DSV3-FP8]: their inputs are quantised in 1x128 tiles like the forward
// activations).  Three kernels; the dgrad GEMMs themselves are the grouped
// GEMM of gemm.hip with the transposed weights as B.
//
// combine backward: for y[t] = sum_k gate[t,k] * c2[dst_row[t,k]] (+ shared),
//   dc2[dst_row[t,k]] = fl32(gate[t,k] * dy[t]), quantised in 1x128 tiles
//   along H (the FP8 operand of the down-projection dgrad), and
//   d_gate[t,k] = <dy[t], c2[dst_row[t,k]]>.  One workgroup per token: the
//   token's dy row is read once and reused for its K slots; each lane owns 8
//   columns per pass (16 lanes per 1x128 tile), the tile amax is a 16-lane
//   shuffle reduction.  The dot products are summed per lane in column order,
//   then across the workgroup in a fixed tree (reproducible).
//
// SwiGLU backward: with g, u the halves of the forward's float32 gate|up row
//   and s the specified sigmoid (device_common.h), in binary32:
//     silu = g * s;  dsilu = s * (1 + g * (1 - s))
//     du = dh * silu;  dg = (dh * u) * dsilu
//   then [dg | du] is quantised in 1x128 tiles along 2I.  32 lanes own one
//   128-wide tile of dh (4 values each) and write one tile of dg and one of
//   du.
//
// router backward: gradient of the gates with respect to the router logits,
//   through the selected experts only (top-K is piecewise constant; the
//   balancing bias selects but does not weight, [DSV3-MOE]).  One wavefront
//   per token, float64 inside, float32 out:
//     sigmoid:  s_k = sigmoid(l_k); normalised gates g_k = s_k / S give
//               dL/ds_k = (dg_k - sum_j dg_j g_j) / S (else dL/ds_k = dg_k);
//               dL/dl = dL/ds_k * s_k (1 - s_k) at the selected experts.
//     softmax:  p = softmax(l) over all E ([PANGU-MOGE]); g_k = p_{e_k};
//               dL/dl_j = p_j (D_j - sum_k dg_k g_k), D_j = dg_k at j = e_k.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

constexpr int kMaxK = 16;  // slots per token held in registers by the combine backward

__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t* __restrict__ dy, const float* __restrict__ y_perm, const int* __restrict__ dst_row,
    const float* __restrict__ gate, int K, int H, uint8_t* __restrict__ dq, float* __restrict__ ds,
    float* __restrict__ d_gate, float* __restrict__ gate_row) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n_rows = (int64_t)gridDim.x * K;  // T * K grouped rows
  auto row_of = [&](int k) {                        // dst_row clamped into range
    const int64_t r = dst_row[t * K + k];
    return r < 0 ? (int64_t)0 : (r >= n_rows ? n_rows - 1 : r);
  };
  if (gate_row && tid < K) gate_row[row_of(tid)] = gate[t * K + tid];
  float part[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) part[k] = 0.f;
  const int nv = H / 8;  // 8-column vectors per row
  for (int v0 = 0; v0 < nv; v0 += blockDim.x) {
    const int v = v0 + tid;
    const bool ok = v < nv;
    float d[8];
    {
      uint4 raw = ok ? *reinterpret_cast<const uint4*>(dy + t * H + 8 * v) : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d[2 * i] = __uint_as_float(w[i] << 16);
        d[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k < K) {  // uniform
        const int64_t r = row_of(k);
        const float g = gate[t * K + k];
        float p[8];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = g * d[i];
          amax = fmaxf(amax, fabsf(p[i]));
        }
        amax = group_max<16>(amax);  // the 16 lanes of one 1x128 tile (whole wave participates)
        if (ok) {
          const float4 y0 = *reinterpret_cast<const float4*>(y_perm + r * H + 8 * v);
          const float4 y1 = *reinterpret_cast<const float4*>(y_perm + r * H + 8 * v + 4);
          const float yy[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) part[k] = part[k] + d[i] * yy[i];
          const float s = scale_from_amax(amax);
          const Divider div(s);
          uint2 c;
          c.x = quantize4(div, p[0], p[1], p[2], p[3]);
          c.y = quantize4(div, p[4], p[5], p[6], p[7]);
          *reinterpret_cast<uint2*>(dq + r * H + 8 * v) = c;
          if ((v & 15) == 0) ds[r * (H / 128) + v / 16] = s;
        }
      }
    }
  }
  // d_gate[t, k]: per-wave butterfly sums, then the 4 waves in order
  __shared__ float red[4][kMaxK];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k < K) {
      float x = part[k];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) x = x + __shfl_xor(x, m, 64);
      if (lane == 0) red[wave][k] = x;
    }
  }
  __syncthreads();
  if (tid < K) d_gate[t * K + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

__global__ __launch_bounds__(256) void swiglu_backward_kernel(const float* __restrict__ gu,
                                                              const float* __restrict__ dh, int64_t M,
                                                              int I, uint8_t* __restrict__ dq,
                                                              float* __restrict__ ds,
                                                              float* __restrict__ d_out) {
  const int64_t nvec = M * (int64_t)(I / 4);  // 4 values of dh per lane
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int qv = I / 4;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v - threadIdx.x % 64 < nvec;
       v += stride) {
    const bool ok = v < nvec;
    float dg[4] = {0.f, 0.f, 0.f, 0.f}, du[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t m = 0;
    int c4 = 0;
    if (ok) {
      m = v / qv;
      c4 = (int)(v % qv);
      const float4 g4 = *reinterpret_cast<const float4*>(gu + m * 2 * I + 4 * c4);
      const float4 u4 = *reinterpret_cast<const float4*>(gu + m * 2 * I + I + 4 * c4);
      const float4 h4 = *reinterpret_cast<const float4*>(dh + m * I + 4 * c4);
      const float g[4] = {g4.x, g4.y, g4.z, g4.w}, u[4] = {u4.x, u4.y, u4.z, u4.w};
      const float d[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = spec_sigmoid(g[i]);
        const float silu = g[i] * s;
        float tt = 1.0f - s;
        tt = g[i] * tt;
        tt = 1.0f + tt;
        const float dsilu = s * tt;
        du[i] = d[i] * silu;
        dg[i] = (d[i] * u[i]) * dsilu;
      }
    }
    float ag = fmaxf(fmaxf(fabsf(dg[0]), fabsf(dg[1])), fmaxf(fabsf(dg[2]), fabsf(dg[3])));
    float au = fmaxf(fmaxf(fabsf(du[0]), fabsf(du[1])), fmaxf(fabsf(du[2]), fabsf(du[3])));
    ag = group_max<32>(ag);
    au = group_max<32>(au);
    if (ok) {
      const float sg = scale_from_amax(ag), su = scale_from_amax(au);
      const int nb = 2 * I / 128;
      *reinterpret_cast<uint32_t*>(dq + m * 2 * I + 4 * c4) = quantize4(Divider(sg), dg[0], dg[1], dg[2], dg[3]);
      *reinterpret_cast<uint32_t*>(dq + m * 2 * I + I + 4 * c4) =
          quantize4(Divider(su), du[0], du[1], du[2], du[3]);
      if ((c4 & 31) == 0) {
        ds[m * nb + c4 / 32] = sg;
        ds[m * nb + I / 128 + c4 / 32] = su;
      }
      if (d_out) {
        *reinterpret_cast<float4*>(d_out + m * 2 * I + 4 * c4) = make_float4(dg[0], dg[1], dg[2], dg[3]);
        *reinterpret_cast<float4*>(d_out + m * 2 * I + I + 4 * c4) = make_float4(du[0], du[1], du[2], du[3]);
      }
    }
  }
}

// One wavefront per token.  Lanes 0..K-1 own the selected slots and write
// their experts' entries; every lane then writes the entries of the
// unselected experts e = lane + 64 i (0, or -p_e * sum_k dg_k g_k for the
// softmax), so each element is written exactly once.
__global__ __launch_bounds__(256) void route_backward_kernel(const float* __restrict__ logits,
                                                             const int* __restrict__ topk_idx,
                                                             const float* __restrict__ d_gate, int T,
                                                             int E, int K, int softmax, int normalize,
                                                             float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits; no barriers below
  const float* row = logits + (int64_t)t * E;
  const int* sel = topk_idx + (int64_t)t * K;
  float* out = d_logits + (int64_t)t * E;
  // softmax max and denominator (float64) over the whole row
  double mx = -1.0e300, sum = 0.0;
  if (softmax) {
    for (int e = lane; e < E; e += 64) mx = fmax(mx, (double)row[e]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mx = fmax(mx, __shfl_xor(mx, m, 64));
    for (int e = lane; e < E; e += 64) sum += exp((double)row[e] - mx);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
  }
  // this lane's slot: its score s (sigmoid, or the softmax probability)
  int e_k = -1;
  double dg = 0.0, s = 0.0;
  if (lane < K) {
    e_k = sel[lane];
    if (e_k >= 0 && e_k < E) {
      dg = (double)d_gate[(int64_t)t * K + lane];
      const double l = (double)row[e_k];
      s = softmax ? exp(l - mx) / sum : 1.0 / (1.0 + exp(-l));
    } else {
      e_k = -1;  // out-of-range id: contributes nothing, written nowhere
    }
  }
  double S = s;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) S += __shfl_xor(S, m, 64);
  const double gk = (softmax || !normalize) ? s : s / S;  // this slot's gate
  double gdot = dg * gk;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) gdot += __shfl_xor(gdot, m, 64);
  if (e_k >= 0) {
    const double v = softmax ? s * (dg - gdot) : (normalize ? (dg - gdot) / S : dg) * s * (1.0 - s);
    out[e_k] = (float)v;
  }
  for (int e = lane; e < E; e += 64) {
    bool chosen = false;
    for (int k = 0; k < K; ++k) chosen |= sel[k] == e;
    if (!chosen) out[e] = softmax ? (float)(-(exp((double)row[e] - mx) / sum) * gdot) : 0.0f;
  }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_combine_backward(const uint16_t* dy_bf16, const float* y_perm, const int32_t* dst_row,
                                           const float* topk_gate, int32_t T, int32_t K, int32_t H,
                                           uint8_t* dq, float* ds, float* d_gate, float* gate_row,
                                           void* stream) {
  clear_detail();
  MOE_REQUIRE(T >= 0 && K >= 1 && H > 0 && H % 128 == 0, MOE_ERR_SHAPE,
              "T=%d K=%d H=%d (H a positive multiple of 128)", T, K, H);
  MOE_REQUIRE(K <= kMaxK, MOE_ERR_UNSUPPORTED, "K=%d > %d", K, kMaxK);
  MOE_REQUIRE(elems_ok((int64_t)T * K, H), MOE_ERR_UNSUPPORTED, "T*K=%lld x H=%d above 2^40 elements",
              (long long)T * K, H);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dy_bf16 && y_perm && dst_row && topk_gate && dq && ds && d_gate, MOE_ERR_NULL,
              "every array is required");
  MOE_REQUIRE(aligned(dy_bf16, 16) && aligned(y_perm, 16) && aligned(dq, 8) && aligned(ds, 4) &&
                  aligned(dst_row, 4) && aligned(topk_gate, 4) && aligned(d_gate, 4) && aligned(gate_row, 4),
              MOE_ERR_ALIGN, "dy and y_perm need 16-byte alignment, dq 8-byte");
  hipStream_t st = as_stream(stream);
  combine_backward_kernel<<<(unsigned)T, 256, 0, st>>>(dy_bf16, y_perm, dst_row, topk_gate, K, H, dq, ds,
                                                       d_gate, gate_row);
  return after_launch("moe_combine_backward", st);
}

extern "C" moe_status swiglu_backward(const float* gate_up, const float* dh, int64_t M, int32_t I, uint8_t* dq,
                                      float* ds, float* d, void* stream) {
  clear_detail();
  MOE_REQUIRE(M >= 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "M=%lld I=%d (I a positive multiple of 128)",
              (long long)M, I);
  MOE_REQUIRE(elems_ok(M, 2 * (int64_t)I), MOE_ERR_UNSUPPORTED, "M=%lld x 2I=%lld above 2^40 elements",
              (long long)M, 2 * (long long)I);
  if (M == 0) return MOE_OK;
  MOE_REQUIRE(gate_up && dh && dq && ds, MOE_ERR_NULL, "gate_up, dh, dq and ds are required");
  MOE_REQUIRE(aligned(gate_up, 16) && aligned(dh, 16) && aligned(dq, 4) && aligned(ds, 4) && aligned(d, 16),
              MOE_ERR_ALIGN, "gate_up, dh and d need 16-byte alignment");
  hipStream_t st = as_stream(stream);
  const int64_t nvec = M * (I / 4);
  const int64_t need = (nvec + 255) / 256;
  swiglu_backward_kernel<<<(unsigned)(need < 16384 ? need : 16384), 256, 0, st>>>(gate_up, dh, M, I, dq, ds, d);
  return after_launch("swiglu_backward", st);
}

extern "C" moe_status moe_route_backward(const float* logits, const int32_t* topk_idx, const float* d_gate,
                                         int32_t T, int32_t E, int32_t K, moe_route_mode mode,
                                         int32_t normalize_topk, float* d_logits, void* stream) {
  clear_detail();
  MOE_REQUIRE(mode == MOE_ROUTE_SIGMOID_BIAS || mode == MOE_ROUTE_SOFTMAX_GROUPED, MOE_ERR_UNSUPPORTED,
              "mode %d", (int)mode);
  MOE_REQUIRE(T >= 0 && E >= 1 && K >= 1 && K <= E, MOE_ERR_SHAPE, "T=%d E=%d K=%d", T, E, K);
  MOE_REQUIRE(K <= 64, MOE_ERR_UNSUPPORTED, "K=%d > 64", K);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(logits && topk_idx && d_gate && d_logits, MOE_ERR_NULL, "every array is required");
  MOE_REQUIRE(aligned(logits, 4) && aligned(topk_idx, 4) && aligned(d_gate, 4) && aligned(d_logits, 4),
              MOE_ERR_ALIGN, "4-byte alignment required");
  hipStream_t st = as_stream(stream);
  route_backward_kernel<<<(unsigned)(((int64_t)T + 3) / 4), 256, 0, st>>>(
      logits, topk_idx, d_gate, T, E, K, mode == MOE_ROUTE_SOFTMAX_GROUPED ? 1 : 0, normalize_topk, d_logits);
  return after_launch("moe_route_backward", st);
}
