// Device helpers shared by the gfx950 kernels of libmoefp8: the E4M3FN
// encoder, the binary32 sigmoid specification, bf16 rounding and wave-level
// reductions.  Everything here is written for 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moefp8 {

constexpr float kE4M3Max = 448.0f;

// 16-byte global accesses that bypass the caches' normal retention policy
// (streamed data that is touched once).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// FP8 quantisation: code = RNE_E4M3(clamp(fl32(x / s), -448, 448)).
//
// Division.  fl32(x / s) is the correctly rounded quotient.  It is formed
// with Markstein's FMA correction (P. Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1),
// 1990): with r = RN(1/s) and the faithful quotient q0 = RN(x * r), the
// residual x - s * q0 is exact in one FMA and RN(q0 + residual * r) equals
// RN(x / s).  The theorem needs r and the residual free of overflow and
// underflow; the scales here are fl32(amax / 448), so the correction is used
// for s >= 2^-100 (r normal, quotients at most ~448) and a direct correctly
// rounded division otherwise.  A zero quotient takes the sign of x.
//
// Encoding.  gfx950's V_CVT_PK_FP8_F32 converts two binary32 values to OCP
// E4M3FN (bias 7, 3 mantissa bits, max 448) with round to nearest-even,
// including the subnormal codes; inputs are clamped to +-448 first.
// ---------------------------------------------------------------------------
struct Divider {
  float s, r;
  bool direct;  // wave-uniform: some active lane's scale is below 2^-100
  __device__ __forceinline__ explicit Divider(float s_)
      : s(s_), r(1.0f / s_), direct(__builtin_amdgcn_ballot_w64(s_ < 0x1p-100f) != 0) {}
  template <bool kDirect>
  __device__ __forceinline__ float div(float x) const {
    if (kDirect) return x / s;
    const float q0 = x * r;
    const float e = __builtin_fmaf(-s, q0, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
  }
};

// Scale of a tile or block from its amax: fl32(amax / 448), 1 if amax == 0.
__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

__device__ __forceinline__ float clamp_e4m3(float y) { return fminf(fmaxf(y, -kE4M3Max), kE4M3Max); }

// Codes of four values under one scale, packed little-endian (x0 in the low
// byte), as stored in the row-major code arrays.
template <bool kDirect>
__device__ __forceinline__ uint32_t quantize4_impl(const Divider& d, float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(d.div<kDirect>(x0)), clamp_e4m3(d.div<kDirect>(x1)), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(d.div<kDirect>(x2)), clamp_e4m3(d.div<kDirect>(x3)), w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ uint32_t quantize4(const Divider& d, float x0, float x1, float x2, float x3) {
  return __builtin_expect(d.direct, 0) ? quantize4_impl<true>(d, x0, x1, x2, x3)
                                       : quantize4_impl<false>(d, x0, x1, x2, x3);
}

// ---------------------------------------------------------------------------
// Binary32 sigmoid specification.  Each line is one correctly rounded
// binary32 operation (this library is compiled with -ffp-contract=off and
// correctly rounded division, so a*b+c stays two roundings):
//   E(y): y = clamp(y, -80, 80); n = rint(y * log2(e));
//         r = (y - n*LN2_HI) - n*LN2_LO          (Cody & Waite reduction)
//         p = Horner(1/k!, k = 7..0) at r;  E = p * 2^n
//   sigmoid(x) = 1 / (1 + E(-x));  silu(x) = x * sigmoid(x)
// LN2_HI is binary32 ln 2 with its 9 low significand bits cleared (so
// n*LN2_HI is exact for |n| <= 128), LN2_LO = fl32(ln 2 - LN2_HI); the
// Taylor coefficients are the binary32 roundings of 1/k!.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float spec_exp(float y) {
  constexpr float kLog2e = 0x1.715476p+0f;
  constexpr float kLn2Hi = 0x1.62e4p-1f;
  constexpr float kLn2Lo = 0x1.7f7d1cp-20f;
  constexpr float c7 = 0x1.a01a02p-13f, c6 = 0x1.6c16c2p-10f, c5 = 0x1.111112p-7f,
                  c4 = 0x1.555556p-5f, c3 = 0x1.555556p-3f, c2 = 0x1p-1f, c1 = 0x1p+0f,
                  c0 = 0x1p+0f;
  y = fminf(fmaxf(y, -80.0f), 80.0f);
  const float n = __builtin_rintf(y * kLog2e);
  const float r = (y - n * kLn2Hi) - n * kLn2Lo;
  float p = c7;
  p = p * r + c6;
  p = p * r + c5;
  p = p * r + c4;
  p = p * r + c3;
  p = p * r + c2;
  p = p * r + c1;
  p = p * r + c0;
  const float two_n = __int_as_float(((int)n + 127) << 23);
  return p * two_n;
}

__device__ __forceinline__ float spec_sigmoid(float x) { return 1.0f / (1.0f + spec_exp(-x)); }

__device__ __forceinline__ float spec_silu(float x) { return x * spec_sigmoid(x); }

// bf16 bit pattern of a finite binary32 value, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Max over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Transposed write of one 128x128-byte block held in LDS (row pitch
// kTilePitch bytes, as 32-bit words): each of 256 threads gathers a
// 16-row x 4-column byte patch with 16 dword reads, transposes it in
// registers with shifts and masks, and writes 4 output rows of 16 bytes
// (8 lanes per 128-byte output row segment).  dst points at the block's first
// output byte, dst_ld is the output row stride.  The pitch of 132 bytes
// spreads the column-wise dword reads over the LDS banks.
// ---------------------------------------------------------------------------
constexpr int kTilePitch = 132;

__device__ __forceinline__ void write_block_transposed(const uint32_t* tile, uint8_t* dst, int64_t dst_ld,
                                                       int tid) {
  const int r0 = 16 * (tid & 7);
  const int c0 = 4 * (tid >> 3);
  uint32_t d[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) d[j] = tile[((r0 + j) * kTilePitch + c0) / 4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t o[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t sh = 8 * i;
      o[jj] = ((d[4 * jj] >> sh) & 0xffu) | (((d[4 * jj + 1] >> sh) & 0xffu) << 8) |
              (((d[4 * jj + 2] >> sh) & 0xffu) << 16) | (((d[4 * jj + 3] >> sh) & 0xffu) << 24);
    }
    store16_nt(dst + (int64_t)(c0 + i) * dst_ld + r0, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

}  // namespace moefp8
