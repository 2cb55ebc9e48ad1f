// Per-token routing as wavefront device functions, shared by the routing
// kernel and the single-launch routing + permutation kernel.
//
// SIGMOID_BIAS ([DSV3-MOE], section 2.1): sigmoid affinity per expert, a
// per-expert bias shifts the selection key, the K best keys win (lower
// expert index on equal keys), gates are the unbiased sigmoid scores,
// optionally normalised over the K winners in slot order.
// SOFTMAX_GROUPED ([PANGU-MOGE], grouped expert selection): experts in G
// equal groups, each group keeps its K' largest logits (equivalently its K'
// largest softmax scores), gates are the global softmax scores (float64 on
// the device, rounded once to float32).
//
// One 64-lane wavefront routes one token.  Each lane keeps the keys of
// experts e = lane + 64*i in registers (E <= 1024 -> at most 16 per lane).
// Every pick is a wave-wide arg-max on (key, -index) by butterfly shuffles,
// so K picks cost K reductions and no memory traffic beyond the logits row.
// The lane that writes slot k's expert also calls on_pick(k, expert) (the
// single-launch routing + permutation counts and marks its picks there).
#pragma once

#include "device_common.h"

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

struct NoPick {
  __device__ void operator()(int, int) const {}
};

// Sigmoid + bias top-K of one token's logits row; writes idx[0..K) and
// gate[0..K).  Called by all 64 lanes of a wave (no barriers inside).
template <int PL, class OnPick = NoPick>
__device__ __forceinline__ void route_sigmoid_token(const float* __restrict__ row, const float* __restrict__ bias,
                                                    int E, int K, int normalize, int* __restrict__ idx,
                                                    float* __restrict__ gate, OnPick on_pick = OnPick{}) {
  const int lane = threadIdx.x & 63;
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
      idx[k] = slot_e[i];
      gate[k] = normalize ? slot_s[i] / total : slot_s[i];
      on_pick(k, slot_e[i]);
    }
  }
}

// Grouped softmax top-K' per group of one token's logits row; writes
// idx[0..G*K') and gate[0..G*K').
template <int PL, class OnPick = NoPick>
__device__ __forceinline__ void route_grouped_token(const float* __restrict__ row, int E, int G, int Kp,
                                                    int* __restrict__ idx, float* __restrict__ gate,
                                                    OnPick on_pick = OnPick{}) {
  const int lane = threadIdx.x & 63;
  const int per = E / G;
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
        idx[k] = c.e;
        gate[k] = (float)(__hiloint2double(zhi, zlo) / sum);
        on_pick(k, c.e);
      }
    }
  }
}

// Host-side dispatch on the number of expert keys per lane.
template <template <int> class F, typename... A>
void dispatch_per_lane(int E, A... a) {
  const int pl = (E + 63) / 64;
  if (pl <= 1) F<1>::run(a...);
  else if (pl <= 2) F<2>::run(a...);
  else if (pl <= 4) F<4>::run(a...);
  else if (pl <= 8) F<8>::run(a...);
  else F<kMaxPerLane>::run(a...);
}

}  // namespace
}  // namespace moefp8
