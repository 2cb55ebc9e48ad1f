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
// E4M3FN encoding (OCP 8-bit float, bias 7, 3 mantissa bits, max 448).
// Input: finite binary32 with |v| <= 448.  Round to nearest, ties to even,
// sign kept.  Pure integer work on the binary32 pattern:
//  * |v| >= 2^-6 (normal E4M3): keep the top 3 mantissa bits with
//    round-half-even (add 0x7FFFF plus the kept LSB, shift right by 20); the
//    biased exponent moves from bias 127 to bias 7, i.e. subtract
//    (127 - 7) << 3 = 0x3C0 from the (exponent << 3 | mantissa) field.  A
//    mantissa carry rolls into the exponent, which is still correct.
//  * |v| < 2^-6 (subnormal E4M3, spacing 2^-9): |v| * 2^9 is exact and
//    rint (half-even) gives the code directly (0..8; 8 is 2^-6 = 0x08).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  const uint32_t normal = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - 0x3c0u;
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a), 0x1p-6f) * 512.0f);
  return (a < 0x3c800000u ? sub : normal) | sign;
}

// Scale of a tile or block from its amax: fl32(amax / 448), 1 if amax == 0.
__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

// Code of x under scale s: RNE_E4M3(clamp(fl32(x / s), -448, 448)).
__device__ __forceinline__ uint32_t quantize(float x, float s) {
  const float y = fminf(fmaxf(x / s, -kE4M3Max), kE4M3Max);
  return e4m3_encode(y);
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

}  // namespace moefp8
