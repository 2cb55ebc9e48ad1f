// Weight gradients of the expert GEMMs in FP8 ([DSV3-FP8]: most training
// GEMMs, backward ones included, take FP8 operands with fine-grained scaling
// and promoted accumulation).
//
// The reduction of a weight gradient runs over one expert's tokens:
//   dW_g[o, i] = sum over the expert's rows r of dOut[r, o] * In[r, i].
// Both operands are therefore quantised in 128x1 tiles along the token
// dimension: 128 consecutive rows of one expert in one column, each expert's
// rows padded with zero rows to whole tiles (so no tile spans two experts),
// with the 1x128 quantiser's scale and rounding rules.  They are stored
// transposed, [column, padded row] with row stride ld, so that the matrix
// core reads both along the reduction dimension exactly as in the forward
// GEMM; expert g owns the padded rows [P_g, P_{g+1}),
// P_g = sum over g' < g of 128 ceil(M_g' / 128).
//
// padded_offsets_kernel  P from the group offsets (one workgroup, block scan).
// quant128x1_kernel      one workgroup per (128-row tile of one expert, 64
//   columns).  Rows are read with 16-byte loads (4 floats or 8 bf16 per
//   lane) and staged through LDS transposed; 4 lanes per column
//   take the amax of 32 rows each (shuffle reduction) and each lane writes 32
//   codes (two 16-byte stores).  Rows come from x directly, through a row
//   index (gather), optionally times a per-row factor (the combine gate, for
//   the down projection's output gradient), or as h = silu(g) * u of a
//   float32 gate|up row (the forward's binary32 SwiGLU).
// wgrad_kernel           one workgroup per 128x128 output tile of one expert,
//   4 waves of 64x64, 3 waves per SIMD.  The tile's K is the expert's padded
//   row count (one or two 128-row chunks at the DeepSeek-V3 shape), so the
//   kernel streams its output: every chunk is loaded straight into
//   registers (32 bytes per lane and operand fragment; staging through LDS
//   and a persistent tile walk both measured slower, the latter because the
//   single vector-memory counter makes each tile's prefetch wait for the
//   previous tile's stores), multiplied with one
//   V_MFMA_SCALE_F32_16X16X128_F8F6F4 per 16x16 block with a zero
//   accumulator, and promoted with one FMA per output by the product of the
//   two 128x1 scales (which vary along both output axes; stored tile-major,
//   [padded row / 128, column], so a fragment's scales are contiguous).  The
//   input operand sits on the instruction's row axis, so each lane holds 4
//   consecutive input features of one output row and stores them as one
//   16-byte (float32) or 8-byte (bf16) vector.  Tiles of one expert are
//   consecutive and the logical tile order is dealt XCD by XCD; inside an
//   expert the order is blocked (4 output-feature tiles by every
//   input-feature tile), so the tiles in flight on one XCD share a few
//   operand slabs, which stay in its L2 despite the output stream passing
//   through it.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxGroups = 1024;
constexpr int kOB = 4;  // output-feature tiles per block of the wgrad tile order (measured: 1, 2, 4, 8, 16)

__global__ __launch_bounds__(256) void padded_offsets_kernel(const int* __restrict__ offsets, int G,
                                                             int* __restrict__ poff) {
  __shared__ int part[256];
  const int t = threadIdx.x;
  int local[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * t + i;
    int n = 0;
    if (g < G) {
      n = offsets[g + 1] - offsets[g];
      n = n < 0 ? 0 : (n + 127) / 128 * 128;
    }
    local[i] = n;
    sum += n;
  }
  part[t] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan
    const int v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;  // exclusive prefix of this thread's groups
  if (t == 0) poff[0] = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * t + i;
    run += local[i];
    if (g < G) poff[g + 1] = run;
  }
}

// 16 bytes of x as float32 values: 4 floats or 8 bf16.
__device__ __forceinline__ void load16(const float* p, float v[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x, v[1] = f.y, v[2] = f.z, v[3] = f.w;
}
__device__ __forceinline__ void load16(const uint16_t* p, float v[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) v[2 * i] = __uint_as_float(u[i] << 16), v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
}

template <typename XT, bool kSwiglu>
__global__ __launch_bounds__(256) void quant128x1_kernel(
    const XT* __restrict__ x, int64_t ldx, int64_t x_rows, int C, const int* __restrict__ row_index,
    const float* __restrict__ row_scale, const int* __restrict__ offsets, const int* __restrict__ poff, int G,
    int64_t M, int64_t ld, uint8_t* __restrict__ qt, float* __restrict__ st) {
  __shared__ float tile[64][132];
  const int tt = blockIdx.x;
  const int cb = blockIdx.y;
  const int64_t prow = (int64_t)tt * 128;
  if (prow >= poff[G] || prow + 128 > ld) return;  // past the last expert's tiles (uniform)
  // expert g: the largest g with P_g <= prow (empty experts have P_g == P_{g+1})
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= prow) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int64_t r0 = offsets[g] + (prow - poff[g]);
  int64_t nv = offsets[g + 1] - r0;
  nv = nv < 0 ? 0 : (nv > 128 ? 128 : nv);
  const int n_valid = (int)nv;

  const int tid = threadIdx.x;
  {
    // 16-byte loads: VW values per lane (4 floats or 8 bf16), TPR lanes per
    // 64-column row, RPP rows per pass
    constexpr int VW = 16 / sizeof(XT), TPR = 64 / VW, RPP = 256 / TPR;
    const int cq = tid % TPR, lr = tid / TPR;
    const int c = cb * 64 + VW * cq;
#pragma unroll
    for (int p = 0; p < 128 / RPP; ++p) {
      const int j = lr + RPP * p;
      float v[VW];
#pragma unroll
      for (int i = 0; i < VW; ++i) v[i] = 0.f;
      if (j < n_valid) {
        int64_t r = r0 + j;
        r = r < M ? r : M - 1;
        int64_t src = row_index ? (int64_t)row_index[r] : r;
        src = src < 0 ? 0 : (src >= x_rows ? x_rows - 1 : src);
        if constexpr (kSwiglu) {
          float gg[VW], uu[VW];
          load16(x + src * ldx + c, gg);
          load16(x + src * ldx + C + c, uu);
#pragma unroll
          for (int i = 0; i < VW; ++i) v[i] = spec_silu(gg[i]) * uu[i];
        } else {
          load16(x + src * ldx + c, v);
        }
        if (row_scale) {
          const float f = row_scale[r];
#pragma unroll
          for (int i = 0; i < VW; ++i) v[i] = f * v[i];
        }
      }
#pragma unroll
      for (int i = 0; i < VW; ++i) tile[VW * cq + i][j] = v[i];
    }
  }
  __syncthreads();
  const int c = tid >> 2, qq = tid & 3;
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = *reinterpret_cast<const float4*>(&tile[c][32 * qq + 4 * i]);
    v[4 * i] = f.x, v[4 * i + 1] = f.y, v[4 * i + 2] = f.z, v[4 * i + 3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const float s = scale_from_amax(amax);
  const Divider div(s);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = quantize4(div, v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  const int64_t col = (int64_t)cb * 64 + c;
  uint8_t* dst = qt + col * ld + prow + 32 * qq;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  if (qq == 0) st[(int64_t)tt * C + col] = s;
}

__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = (int)a.x, r[1] = (int)a.y, r[2] = (int)a.z, r[3] = (int)a.w;
  r[4] = (int)b.x, r[5] = (int)b.y, r[6] = (int)b.z, r[7] = (int)b.w;
  return r;
}

__device__ __forceinline__ void store4(float* p, const float v[4], bool acc) {
  float4 o = make_float4(v[0], v[1], v[2], v[3]);
  if (acc) {
    const float4 old = *reinterpret_cast<const float4*>(p);
    o.x = v[0] + old.x, o.y = v[1] + old.y, o.z = v[2] + old.z, o.w = v[3] + old.w;
  }
  *reinterpret_cast<float4*>(p) = o;
}
__device__ __forceinline__ void store4(uint16_t* p, const float v[4], bool acc) {
  float a[4] = {v[0], v[1], v[2], v[3]};
  if (acc) {
    const uint2 old = *reinterpret_cast<const uint2*>(p);
    a[0] = a[0] + __uint_as_float(old.x << 16), a[1] = a[1] + __uint_as_float(old.x & 0xffff0000u);
    a[2] = a[2] + __uint_as_float(old.y << 16), a[3] = a[3] + __uint_as_float(old.y & 0xffff0000u);
  }
  uint2 o;
  o.x = bf16_rne_bits(a[0]) | (bf16_rne_bits(a[1]) << 16);
  o.y = bf16_rne_bits(a[2]) | (bf16_rne_bits(a[3]) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}

template <typename OT, bool kAcc>
__global__ __launch_bounds__(256, 3) void wgrad_kernel(const uint8_t* __restrict__ aq, const float* __restrict__ as,
                                                       const uint8_t* __restrict__ bq, const float* __restrict__ bs,
                                                       const int* __restrict__ poff, int Na, int Nb, int64_t ld,
                                                       int64_t n_tiles, int64_t per_xcd, OT* __restrict__ out) {
  const int64_t b = blockIdx.x;
  const int64_t tile = (b & 7) * per_xcd + (b >> 3);  // workgroup b runs on XCD b % 8
  if (tile >= n_tiles) return;
  const int to_n = Na / 128, ti_n = Nb / 128;
  const int64_t per_g = (int64_t)to_n * ti_n;
  const int g = (int)(tile / per_g);
  const int rem = (int)(tile % per_g);
  // blocked order inside the expert: blocks of kOB output-feature tiles, and
  // inside a block the input-feature tile outermost, so the tiles an XCD runs
  // at once share a few operand slabs of each kind instead of one A slab and
  // every B slab (which the output stream would evict before their reuse)
  const int ob = rem / (kOB * ti_n), r2 = rem % (kOB * ti_n);
  const int obs = to_n - ob * kOB < kOB ? to_n - ob * kOB : kOB;  // tiles in this block
  const int to = ob * kOB + r2 % obs, ti = r2 / obs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t i_base = (int64_t)ti * 128 + (wave & 1) * 64;   // input features (instruction rows)
  const int64_t o_base = (int64_t)to * 128 + (wave >> 1) * 64;  // output features (instruction columns)
  const int64_t nkb = ld / 128;
  int64_t kb0 = poff[g] / 128, kb1 = poff[g + 1] / 128;
  kb0 = kb0 < 0 ? 0 : (kb0 > nkb ? nkb : kb0);
  kb1 = kb1 < kb0 ? kb0 : (kb1 > nkb ? nkb : kb1);

  v4f acc[4][4];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int fo = 0; fo < 4; ++fo) acc[fi][fo] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint8_t* pa = bq + (i_base + l16) * ld + 32 * q;  // In rows i_base + 16 f + lane % 16
  const uint8_t* pb = aq + (o_base + l16) * ld + 32 * q;  // dOut rows o_base + 16 f + lane % 16
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    v8i A[4], B[4];
    float sI[4][4], sO[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      A[f] = load_frag(pa + 16 * f * ld + kb * 128);
      B[f] = load_frag(pb + 16 * f * ld + kb * 128);
      // tile-major scales: In rows i_base + 16 f + 4 q + v are contiguous
      const float4 s4 = *reinterpret_cast<const float4*>(bs + kb * Nb + i_base + 16 * f + 4 * q);
      sI[f][0] = s4.x, sI[f][1] = s4.y, sI[f][2] = s4.z, sI[f][3] = s4.w;
      sO[f] = as[kb * Na + o_base + 16 * f + l16];
    }
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int fo = 0; fo < 4; ++fo) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[fi], B[fo], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[fi][fo][v] = __builtin_fmaf(p[v], sI[fi][v] * sO[fo], acc[fi][fo][v]);
      }
  }
  OT* og = out + (int64_t)g * Na * Nb;
#pragma unroll
  for (int fo = 0; fo < 4; ++fo)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      const float v[4] = {acc[fi][fo][0], acc[fi][fo][1], acc[fi][fo][2], acc[fi][fo][3]};
      store4(og + (o_base + 16 * fo + l16) * Nb + i_base + 16 * fi + 4 * q, v, kAcc);
    }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_wgrad_padded_rows(int64_t M, int32_t G, int64_t* rows) {
  clear_detail();
  MOE_REQUIRE(rows, MOE_ERR_NULL, "rows is required");
  MOE_REQUIRE(M >= 0 && G >= 1, MOE_ERR_SHAPE, "M=%lld G=%d", (long long)M, G);
  *rows = 128 * ((M + 127) / 128 + (int64_t)G);
  return MOE_OK;
}

extern "C" moe_status quant_act_128x1_grouped_e4m3(const void* x, moe_dtype x_dtype, int32_t swiglu_input,
                                                   int64_t x_rows, int32_t C, const int32_t* row_index,
                                                   const float* row_scale, const int32_t* group_offsets,
                                                   int32_t G, int64_t M, int64_t ld, int32_t* padded_offsets,
                                                   uint8_t* qt, float* st, void* stream) {
  clear_detail();
  MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "x_dtype %d", (int)x_dtype);
  MOE_REQUIRE(!swiglu_input || x_dtype == MOE_F32, MOE_ERR_UNSUPPORTED, "a gate|up input must be float32");
  MOE_REQUIRE(C > 0 && C % 128 == 0, MOE_ERR_SHAPE, "C=%d (a positive multiple of 128)", C);
  MOE_REQUIRE(G >= 1 && G <= kMaxGroups, MOE_ERR_UNSUPPORTED, "G=%d (1..%d)", G, kMaxGroups);
  MOE_REQUIRE(M >= 0 && x_rows >= 0, MOE_ERR_SHAPE, "M=%lld x_rows=%lld", (long long)M, (long long)x_rows);
  MOE_REQUIRE(row_index || x_rows >= M, MOE_ERR_SHAPE, "without a row index x needs M=%lld rows, has %lld",
              (long long)M, (long long)x_rows);
  MOE_REQUIRE(M == 0 || x_rows >= 1, MOE_ERR_SHAPE, "x has no rows");
  const int64_t need = 128 * ((M + 127) / 128 + (int64_t)G);
  MOE_REQUIRE(ld % 128 == 0 && ld >= need, MOE_ERR_SHAPE,
              "ld=%lld must be a multiple of 128 and at least 128 (ceil(M/128) + G) = %lld", (long long)ld,
              (long long)need);
  MOE_REQUIRE(ld / 128 <= 0x7fffffff, MOE_ERR_UNSUPPORTED, "ld too large");
  MOE_REQUIRE(group_offsets && padded_offsets, MOE_ERR_NULL, "group_offsets and padded_offsets are required");
  MOE_REQUIRE(M == 0 || (x && qt && st), MOE_ERR_NULL, "x, qt and st are required");
  MOE_REQUIRE(aligned(group_offsets, 4) && aligned(padded_offsets, 4) && aligned(x, 16) && aligned(qt, 16) &&
                  aligned(st, 4) && aligned(row_index, 4) && aligned(row_scale, 4),
              MOE_ERR_ALIGN, "x and qt need 16-byte alignment, the others 4-byte");
  hipStream_t s = as_stream(stream);
  padded_offsets_kernel<<<1, 256, 0, s>>>(group_offsets, G, padded_offsets);
  if (M > 0) {
    const dim3 grid((unsigned)((M + 127) / 128 + G), (unsigned)(C / 64));
    const int64_t ldx = swiglu_input ? 2 * (int64_t)C : C;
    if (x_dtype == MOE_F32) {
      if (swiglu_input)
        quant128x1_kernel<float, true><<<grid, 256, 0, s>>>(static_cast<const float*>(x), ldx, x_rows, C,
                                                            row_index, row_scale, group_offsets, padded_offsets,
                                                            G, M, ld, qt, st);
      else
        quant128x1_kernel<float, false><<<grid, 256, 0, s>>>(static_cast<const float*>(x), ldx, x_rows, C,
                                                             row_index, row_scale, group_offsets, padded_offsets,
                                                             G, M, ld, qt, st);
    } else {
      quant128x1_kernel<uint16_t, false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), ldx, x_rows, C,
                                                              row_index, row_scale, group_offsets, padded_offsets,
                                                              G, M, ld, qt, st);
    }
  }
  return after_launch("quant_act_128x1_grouped_e4m3", s);
}

extern "C" moe_status grouped_wgrad_fp8(const uint8_t* aq, const float* as, const uint8_t* bq, const float* bs,
                                        const int32_t* padded_offsets, int32_t G, int32_t Na, int32_t Nb,
                                        int64_t ld, void* c, moe_dtype c_dtype, int32_t accumulate,
                                        void* stream) {
  clear_detail();
  MOE_REQUIRE(c_dtype == MOE_F32 || c_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "c_dtype %d", (int)c_dtype);
  MOE_REQUIRE(Na > 0 && Nb > 0 && Na % 128 == 0 && Nb % 128 == 0, MOE_ERR_SHAPE,
              "Na=%d Nb=%d (positive multiples of 128)", Na, Nb);
  MOE_REQUIRE(G >= 1 && G <= kMaxGroups, MOE_ERR_UNSUPPORTED, "G=%d (1..%d)", G, kMaxGroups);
  MOE_REQUIRE(ld > 0 && ld % 128 == 0, MOE_ERR_SHAPE, "ld=%lld (a positive multiple of 128)", (long long)ld);
  const int64_t n_tiles = (int64_t)G * (Na / 128) * (Nb / 128);
  MOE_REQUIRE(n_tiles <= 0x7fffffffLL - 8, MOE_ERR_UNSUPPORTED, "too many output tiles");
  MOE_REQUIRE(aq && as && bq && bs && padded_offsets && c, MOE_ERR_NULL, "every array is required");
  MOE_REQUIRE(aligned(aq, 16) && aligned(bq, 16) && aligned(as, 4) && aligned(bs, 4) &&
                  aligned(padded_offsets, 4) && aligned(c, c_dtype == MOE_F32 ? 16 : 8),
              MOE_ERR_ALIGN, "aq, bq (and a float32 c) need 16-byte alignment, a bf16 c 8-byte");
  hipStream_t s = as_stream(stream);
  const int64_t per_xcd = (n_tiles + 7) / 8;
  const unsigned grid = (unsigned)(8 * per_xcd);
#define MOE_WGRAD_LAUNCH(OT, ACC)                                                                          \
  wgrad_kernel<OT, ACC><<<grid, 256, 0, s>>>(aq, as, bq, bs, padded_offsets, Na, Nb, ld, n_tiles, per_xcd, \
                                            static_cast<OT*>(c))
  if (c_dtype == MOE_F32) {
    if (accumulate) MOE_WGRAD_LAUNCH(float, true); else MOE_WGRAD_LAUNCH(float, false);
  } else {
    if (accumulate) MOE_WGRAD_LAUNCH(uint16_t, true); else MOE_WGRAD_LAUNCH(uint16_t, false);
  }
#undef MOE_WGRAD_LAUNCH
  return after_launch("grouped_wgrad_fp8", s);
}
