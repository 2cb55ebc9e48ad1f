// FP8 quantisers: 1x128 activation tiles and 128x128 weight blocks of every
// expert in one launch ([KANANA-FP8] all-experts MoE quantisation kernel;
// [DSV3-FP8] tile/block granularity).  Both are single coalesced HBM passes:
// each value is read once and its code written once.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

// Input element access: 16-byte vectors of 8 bf16 or 4 fp32 values.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void unpack(const uint4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec<float> {
  static constexpr int kElems = 4;
  __device__ static void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};

template <int E>
__device__ __forceinline__ void store_codes(uint8_t* dst, const Divider& d, const float* f);
template <>
__device__ __forceinline__ void store_codes<8>(uint8_t* dst, const Divider& d, const float* f) {
  uint2 v;
  v.x = quantize4(d, f[0], f[1], f[2], f[3]);
  v.y = quantize4(d, f[4], f[5], f[6], f[7]);
  *reinterpret_cast<uint2*>(dst) = v;
}
template <>
__device__ __forceinline__ void store_codes<4>(uint8_t* dst, const Divider& d, const float* f) {
  *reinterpret_cast<uint32_t*>(dst) = quantize4(d, f[0], f[1], f[2], f[3]);
}

// ---------------------------------------------------------------------------
// 1x128 tiles.  One lane owns one 16-byte input vector; the 128/kElems lanes
// of a tile (16 for bf16, 32 for fp32, always an aligned lane group) reduce
// their amax with cross-lane shuffles.  Grid-stride over vectors, unrolled so
// that each lane keeps several 16-byte loads in flight.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quant_act_kernel(const T* __restrict__ x, int64_t n_vec,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  constexpr int E = Vec<T>::kElems;
  constexpr int LPT = 128 / E;  // lanes per tile
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  for (int64_t v0 = base; v0 - threadIdx.x % 64 < n_vec; v0 += stride * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * stride;
      raw[u] = v < n_vec ? load16_nt(xv + v) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * stride;
      float f[E];
      Vec<T>::unpack(raw[u], f);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = group_max<LPT>(amax);  // whole wave participates (uniform control)
      if (v < n_vec) {
        const float s = scale_from_amax(amax);
        store_codes<E>(q + v * E, Divider(s), f);
        if ((threadIdx.x % LPT) == 0) scale[v / LPT] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks, one 256-thread workgroup per block (all experts in one
// grid).  Each thread holds its share of the block in registers (32 KB of
// bf16 or 64 KB of fp32 per block), the block amax is reduced in-wave and
// across the 4 waves through LDS, then codes are written from registers.
// Loads are 16-byte vectors; a wave covers whole 256/512-byte row segments.
// ---------------------------------------------------------------------------
template <typename T, bool kT>
__global__ __launch_bounds__(256) void quant_weight_kernel(const T* __restrict__ w, int rows,
                                                           int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale, uint8_t* __restrict__ qt,
                                                           float* __restrict__ scale_t) {
  constexpr int E = Vec<T>::kElems;
  constexpr int VPR = 128 / E;              // vectors per block row
  constexpr int NV = 128 * VPR / 256;       // vectors per thread
  const int bc = cols / 128, br = rows / 128;
  const int64_t blk = blockIdx.x;
  const int bj = (int)(blk % bc);
  const int bi = (int)((blk / bc) % br);
  const int64_t g = blk / ((int64_t)bc * br);
  const int64_t gbase = g * rows * (int64_t)cols;
  const int tid = threadIdx.x;
  uint4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = i * 256 + tid;
    const int r = id / VPR, cv = id % VPR;
    const int64_t off = gbase + (int64_t)(bi * 128 + r) * cols + bj * 128 + cv * E;
    raw[i] = load16_nt(w + off);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float f[E];
    Vec<T>::unpack(raw[i], f);
#pragma unroll
    for (int k = 0; k < E; ++k) amax = fmaxf(amax, fabsf(f[k]));
  }
  amax = group_max<64>(amax);
  __shared__ float red[4];
  __shared__ uint32_t tile[kT ? 128 * kTilePitch / 4 : 1];  // the block's codes, for the transposed copy
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_from_amax(amax);
  const Divider div(s);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = i * 256 + tid;
    const int r = id / VPR, cv = id % VPR;
    const int64_t off = gbase + (int64_t)(bi * 128 + r) * cols + bj * 128 + cv * E;
    float f[E];
    Vec<T>::unpack(raw[i], f);
    uint32_t c[E / 4];
#pragma unroll
    for (int k = 0; k < E / 4; ++k) c[k] = quantize4(div, f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
    if constexpr (E == 8) {
      *reinterpret_cast<uint2*>(q + off) = make_uint2(c[0], c[1]);
    } else {
      *reinterpret_cast<uint32_t*>(q + off) = c[0];
    }
    if constexpr (kT) {
#pragma unroll
      for (int k = 0; k < E / 4; ++k) tile[(r * kTilePitch + cv * E) / 4 + k] = c[k];
    }
  }
  if (tid == 0) scale[blk] = s;  // [G, rows/128, cols/128] row-major == blk order
  if constexpr (kT) {
    // the block transposed: qt [G, cols, rows], scale_t [G, cols/128, rows/128]
    __syncthreads();
    write_block_transposed(tile, qt + gbase + (int64_t)bj * 128 * rows + bi * 128, rows, tid);
    if (tid == 0) scale_t[g * (int64_t)br * bc + (int64_t)bj * br + bi] = s;
  }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status quant_act_1x128_e4m3(const void* x, moe_dtype x_dtype, int64_t rows,
                                           int32_t cols, uint8_t* q, float* scale, void* stream) {
  clear_detail();
  MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "x_dtype %d", (int)x_dtype);
  MOE_REQUIRE(rows >= 0 && cols > 0 && cols % 128 == 0, MOE_ERR_SHAPE,
              "rows=%lld cols=%d (cols must be a positive multiple of 128)", (long long)rows, cols);
  MOE_REQUIRE(elems_ok(rows, cols), MOE_ERR_UNSUPPORTED, "rows=%lld x cols=%d above 2^40 elements",
              (long long)rows, cols);
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(x && q && scale, MOE_ERR_NULL, "x, q and scale are required");
  MOE_REQUIRE(aligned(x, 16) && aligned(q, 16) && aligned(scale, 4), MOE_ERR_ALIGN,
              "x and q need 16-byte alignment, scale 4-byte");
  hipStream_t st = as_stream(stream);
  const int elems = x_dtype == MOE_BF16 ? 8 : 4;
  const int64_t n_vec = rows * (int64_t)cols / elems;
  const int64_t blocks_needed = (n_vec + 255) / 256;
  const unsigned grid = (unsigned)(blocks_needed < 8192 ? blocks_needed : 8192);
  if (x_dtype == MOE_BF16)
    quant_act_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, n_vec, q, scale);
  else
    quant_act_kernel<float><<<grid, 256, 0, st>>>((const float*)x, n_vec, q, scale);
  return after_launch("quant_act_1x128_e4m3", st);
}

namespace moefp8 {
namespace {

moe_status quant_weight_impl(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows, int32_t cols,
                             uint8_t* q, float* scale, uint8_t* qt, float* scale_t, void* stream,
                             const char* what) {
  MOE_REQUIRE(w_dtype == MOE_F32 || w_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "w_dtype %d", (int)w_dtype);
  MOE_REQUIRE(G >= 0 && rows > 0 && cols > 0 && rows % 128 == 0 && cols % 128 == 0, MOE_ERR_SHAPE,
              "G=%d rows=%d cols=%d (rows, cols positive multiples of 128)", G, rows, cols);
  MOE_REQUIRE(elems_ok((int64_t)G * rows, cols), MOE_ERR_UNSUPPORTED, "G=%d x %d x %d above 2^40 elements", G,
              rows, cols);
  if (G == 0) return MOE_OK;
  MOE_REQUIRE(w && q && scale, MOE_ERR_NULL, "w, q and scale are required");
  MOE_REQUIRE(aligned(w, 16) && aligned(q, 16) && aligned(scale, 4) && aligned(qt, 16) && aligned(scale_t, 4),
              MOE_ERR_ALIGN, "w, q and qt need 16-byte alignment, the scales 4-byte");
  const int64_t nblk = (int64_t)G * (rows / 128) * (cols / 128);
  MOE_REQUIRE(nblk < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many blocks (%lld)", (long long)nblk);
  hipStream_t st = as_stream(stream);
#define MOE_QW_LAUNCH(T, TR) \
  quant_weight_kernel<T, TR><<<(unsigned)nblk, 256, 0, st>>>((const T*)w, rows, cols, q, scale, qt, scale_t)
  if (w_dtype == MOE_BF16) {
    if (qt) MOE_QW_LAUNCH(uint16_t, true); else MOE_QW_LAUNCH(uint16_t, false);
  } else {
    if (qt) MOE_QW_LAUNCH(float, true); else MOE_QW_LAUNCH(float, false);
  }
#undef MOE_QW_LAUNCH
  return after_launch(what, st);
}

}  // namespace
}  // namespace moefp8

extern "C" moe_status quant_weight_128x128_e4m3(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows,
                                                int32_t cols, uint8_t* q, float* scale, void* stream) {
  clear_detail();
  return quant_weight_impl(w, w_dtype, G, rows, cols, q, scale, nullptr, nullptr, stream,
                           "quant_weight_128x128_e4m3");
}

extern "C" moe_status quant_weight_128x128_e4m3_t(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows,
                                                  int32_t cols, uint8_t* q, float* scale, uint8_t* qt,
                                                  float* scale_t, void* stream) {
  clear_detail();
  if (G > 0) MOE_REQUIRE(qt && scale_t, MOE_ERR_NULL, "qt and scale_t are required");
  return quant_weight_impl(w, w_dtype, G, rows, cols, q, scale, qt, scale_t, stream,
                           "quant_weight_128x128_e4m3_t");
}
