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
// wgrad_kernel           256x256 output tiles of one expert, 8 waves of 128
//   (input features) x 64 (output features), 2 waves per SIMD, one
//   workgroup per compute unit walking its share of the tiles.  The tile's
//   K is the expert's padded row count (one or two 128-row chunks at the
//   DeepSeek-V3 shape), so the kernel streams its output, and what bounds
//   it is the traffic through each compute unit's vector-memory path
//   (operand loads plus the output).  Each chunk's operand rows and scales
//   go straight from global memory into a 2-stage LDS ring (global_load_lds,
//   no register staging; 128-byte rows with the 16-byte XOR swizzle of the
//   forward GEMM), so a workgroup reads each operand byte once: (256 + 256)
//   x 128 bytes per chunk for 256 x 256 outputs, against twice that per
//   128 x 128 outputs when every wave loads its own fragments.  The ring
//   runs across tile boundaries: the next tile's first chunk is loaded while
//   the current tile is multiplied and stored, and no workgroup launch
//   separates two tiles.  Every chunk is multiplied with one
//   V_MFMA_SCALE_F32_16X16X128_F8F6F4 per 16x16 block with a zero
//   accumulator and promoted with one FMA per output by the product of the
//   two 128x1 scales (which vary along both output axes; stored tile-major,
//   [padded row / 128, column], so a chunk's scales are contiguous).  The
//   input operand sits on the instruction's row axis, so each lane holds 4
//   consecutive input features of one output row and stores them as one
//   16-byte float32 vector; for bf16 output two lanes trade halves first
//   (a lane-row swap), so each lane still stores 16 bytes and each store
//   writes 64 contiguous bytes of a row.  Tiles of one expert are
//   consecutive and the logical tile order is dealt XCD by XCD; inside an
//   expert the order is blocked (2 output-feature tiles by every
//   input-feature tile), so the tiles in flight on one XCD share a few
//   operand slabs, which stay in its L2 despite the output stream passing
//   through it, and write long contiguous runs of the same output rows.
#include "host_common.h"
#include "lds_dma.h"

namespace moefp8 {
namespace {

constexpr int kMaxGroups = 1024;
constexpr int kOB = 2;  // output-feature tiles per block of the wgrad tile order (measured: 1, 2, 4, 8)

// wgrad_kernel: 256 x 256 output tiles, 8 waves, a 2-stage LDS ring
constexpr int kWgThreads = 512;
constexpr int kWgTile = 256;
constexpr int kWgOffIn = 0;                              // [256 In rows][128 B]
constexpr int kWgOffOut = kWgTile * 128;                 // [256 Out rows][128 B]
constexpr int kWgOffSIn = 2 * kWgTile * 128;             // [256] float In scales
constexpr int kWgOffSOut = kWgOffSIn + 4 * kWgTile;      // [256] float Out scales
constexpr int kWgStageBytes = kWgOffSOut + 4 * kWgTile;  // 67584; 2 stages = 135168 B of LDS
constexpr int kWgDmaPerChunk = 9;                        // per wave: 4 + 4 row slices, 1 scale slice

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
  // [column][row]; a row index is stored XOR 4 ((column / 8) % 8), which
  // keeps every aligned group of 4 rows contiguous (the float4 reads below)
  // and spreads the transposing 4-byte writes of a wave over all 32 banks
  // (2 lanes per bank instead of 8)
  __shared__ float tile[64][132];
  // column blocks fastest: consecutive workgroups read adjacent 128-byte
  // pieces of the same source rows (measured 5-10 % faster than row tiles
  // fastest, whose writes are the contiguous ones)
  const int ncb = C / 64;
  const int tt = (int)(blockIdx.x / ncb);
  const int cb = (int)(blockIdx.x % ncb);
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
      for (int i = 0; i < VW; ++i) tile[VW * cq + i][j ^ (4 * (((VW * cq + i) >> 3) & 7))] = v[i];
    }
  }
  __syncthreads();
  const int c = tid >> 2, qq = tid & 3;
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = *reinterpret_cast<const float4*>(&tile[c][(32 * qq + 4 * i) ^ (4 * ((c >> 3) & 7))]);
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

__device__ __forceinline__ void store4(float* p, const float v[4], bool acc) {
  float4 o = make_float4(v[0], v[1], v[2], v[3]);
  if (acc) {
    const float4 old = *reinterpret_cast<const float4*>(p);
    o.x = v[0] + old.x, o.y = v[1] + old.y, o.z = v[2] + old.z, o.w = v[3] + old.w;
  }
  *reinterpret_cast<float4*>(p) = o;
}
// 8 consecutive bf16 outputs (one 16-byte store), optionally added to the
// values already there (each sum rounded once to bf16).
__device__ __forceinline__ void store8(uint16_t* p, const float v[8], bool acc) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = v[i];
  if (acc) {
    const uint4 old = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = a[2 * i] + __uint_as_float(w[i] << 16);
      a[2 * i + 1] = a[2 * i + 1] + __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  uint4 o;
  o.x = bf16_rne_bits(a[0]) | (bf16_rne_bits(a[1]) << 16);
  o.y = bf16_rne_bits(a[2]) | (bf16_rne_bits(a[3]) << 16);
  o.z = bf16_rne_bits(a[4]) | (bf16_rne_bits(a[5]) << 16);
  o.w = bf16_rne_bits(a[6]) | (bf16_rne_bits(a[7]) << 16);
  *reinterpret_cast<uint4*>(p) = o;
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

template <typename OT, bool kAcc, bool kPair>
__global__ __launch_bounds__(kWgThreads, 2) void wgrad_kernel(const uint8_t* __restrict__ aq,
                                                             const float* __restrict__ as,
                                                             const uint8_t* __restrict__ bq,
                                                             const float* __restrict__ bs,
                                                             const int* __restrict__ poff, int Na, int Nb,
                                                             int64_t ld, int64_t n_tiles, int64_t per_xcd,
                                                             int nwg, OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kWgStageBytes];
  // XCD x (workgroup b runs on XCD b % 8) owns the logical tiles
  // [x per_xcd, (x + 1) per_xcd); its nwg workgroups take every nwg-th one,
  // so the tiles in flight on an XCD stay a window of about nwg neighbours
  const int64_t b = blockIdx.x;
  const int64_t xcd = b & 7;
  const int64_t t_first = xcd * per_xcd + (b >> 3);
  const int64_t t_end = (xcd + 1) * per_xcd < n_tiles ? (xcd + 1) * per_xcd : n_tiles;
  const int to_n = (Na + kWgTile - 1) / kWgTile, ti_n = (Nb + kWgTile - 1) / kWgTile;
  const int64_t per_g = (int64_t)to_n * ti_n;
  const int64_t nkb = ld / 128;
  // tile -> expert, origin and chunk range.  Blocked order inside the
  // expert: blocks of kOB output-feature tiles, and inside a block the
  // input-feature tile outermost, so the tiles an XCD runs at once share a
  // few operand slabs of each kind instead of one A slab and every B slab
  // (which the output stream would evict before their reuse)
  auto decode = [&](int64_t tile, int& g, int& o0, int& i0, int64_t& kb0, int& nk) {
    g = (int)(tile / per_g);
    const int rem = (int)(tile % per_g);
    const int ob = rem / (kOB * ti_n), r2 = rem % (kOB * ti_n);
    const int obs = to_n - ob * kOB < kOB ? to_n - ob * kOB : kOB;  // tiles in this block
    o0 = (ob * kOB + r2 % obs) * kWgTile;
    i0 = (r2 / obs) * kWgTile;
    int64_t k0 = poff[g] / 128, k1 = poff[g + 1] / 128;
    k0 = k0 < 0 ? 0 : (k0 > nkb ? nkb : k0);
    k1 = k1 < k0 ? k0 : (k1 > nkb ? nkb : k1);
    kb0 = k0;
    nk = (int)(k1 - k0);
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform wave index
  const int q = lane >> 4, l16 = lane & 15;

  // ---- issue side: wave w fetches In rows and Out rows 32w .. 32w + 31 of
  // the tile (4 slices of 8 rows each) and one scale slice; rows past Nb / Na
  // re-read the last row.  Lane: row 8j + lane / 8 of slice j, physical
  // 16-byte piece lane % 8, holding the swizzled logical piece.  Scales:
  // waves 0-3 fetch In scales 64w .., waves 4-7 Out scales 64(w - 4) ..
  const int rsub = lane >> 3, c16 = (lane & 7) ^ rsub;
  const bool s_in = w < 4;
  const int s_n = s_in ? Nb : Na;
  const uint32_t s_lds = (s_in ? kWgOffSIn : kWgOffSOut) + 256 * (w & 3);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  auto issue = [&](int o0, int i0, int64_t kb, int stage) {
    const uint32_t st = ring_lds + stage * kWgStageBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * w + 8 * j;
      const int ri = min(i0 + r, Nb - 1);  // scalar: the slice's first (clamped) row
      const uint32_t off = (uint32_t)((int64_t)(min(i0 + r + rsub, Nb - 1) - ri) * ld + c16 * 16);
      dma16(bq + (int64_t)ri * ld + kb * 128, off, st + kWgOffIn + (4 * w + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * w + 8 * j;
      const int ro = min(o0 + r, Na - 1);
      const uint32_t off = (uint32_t)((int64_t)(min(o0 + r + rsub, Na - 1) - ro) * ld + c16 * 16);
      dma16(aq + (int64_t)ro * ld + kb * 128, off, st + kWgOffOut + (4 * w + j) * 1024);
    }
    const int sr = (s_in ? i0 : o0) + 64 * (w & 3);
    const int s_first = min(sr, s_n - 1);
    const uint32_t s_off = (uint32_t)(min(sr + lane, s_n - 1) - s_first) * 4u;
    dma4((s_in ? bs : as) + s_first + kb * s_n, s_off, st + s_lds);
  };
  // The workgroup's chunk stream is its tiles' chunks in order; the issue
  // cursor (tile it, chunk ikb) runs one chunk ahead of the multiplies, so a
  // tile's first chunk is in flight while the previous tile is multiplied
  // and stored.  Tiles of experts without rows have no chunks.
  int64_t it = t_first, ikb = 0, ikb_end = 0;
  int io0 = 0, ii0 = 0;
  auto seek = [&]() {
    for (; it < t_end; it += nwg) {
      int g, nk;
      int64_t kb0;
      decode(it, g, io0, ii0, kb0, nk);
      if (nk > 0) {
        ikb = kb0, ikb_end = kb0 + nk;
        return;
      }
    }
  };
  auto issue_next = [&](int stage) {
    if (it >= t_end) return;
    issue(io0, ii0, ikb, stage);
    if (++ikb == ikb_end) {
      it += nwg;
      seek();
    }
  };
  seek();
  issue_next(0);

  // ---- multiply side: wave w owns In rows wi .. wi + 127 (instruction rows,
  // 8 fragments) by Out rows wo .. wo + 63 (instruction columns, 4 fragments)
  const int wi = (w & 1) * 128, wo = (w >> 1) * 64;
  const uint32_t lane_lo = frag_lane_lo(lane), lane_hi = lane_lo ^ 16;
  v4f acc[8][4];
#pragma unroll
  for (int fi = 0; fi < 8; ++fi)
#pragma unroll
    for (int fo = 0; fo < 4; ++fo) acc[fi][fo] = v4f{0.f, 0.f, 0.f, 0.f};
  int qs = 0;  // position in the chunk stream; its ring stage is qs & 1
  for (int64_t tile = t_first; tile < t_end; tile += nwg) {
    int g, o0, i0, nk;
    int64_t kb0;
    decode(tile, g, o0, i0, kb0, nk);
    for (int c = 0; c < nk; ++c, ++qs) {
      // this wave's loads of chunk qs (its only DMA in flight) have landed
      // and its reads of chunk qs - 1 are done; after the barrier the same
      // holds for every wave, so chunk qs + 1 may take chunk qs - 1's stage.
      // The asm's memory clobber keeps the LDS reads below on this side.
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue_next((qs + 1) & 1);
      const uint8_t* st = ring + (qs & 1) * kWgStageBytes;
      const float* sSI = reinterpret_cast<const float*>(st + kWgOffSIn);
      const float* sSO = reinterpret_cast<const float*>(st + kWgOffSOut);
      v8i bo[4];
      float so[4];
#pragma unroll
      for (int fo = 0; fo < 4; ++fo) {
        bo[fo] = lds_operand(st + kWgOffOut + (wo + 16 * fo) * 128, lane_lo, lane_hi);
        so[fo] = sSO[wo + 16 * fo + l16];
      }
#pragma unroll
      for (int fi = 0; fi < 8; ++fi) {
        const v8i ai = lds_operand(st + kWgOffIn + (wi + 16 * fi) * 128, lane_lo, lane_hi);
        // In rows wi + 16 fi + 4q + v: four consecutive scales
        const float4 s4 = *reinterpret_cast<const float4*>(sSI + wi + 16 * fi + 4 * q);
        const float si[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int fo = 0; fo < 4; ++fo) {
          const v4f p = mfma_chunk(ai, bo[fo]);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[fi][fo][v] = __builtin_fmaf(p[v], si[v] * so[fo], acc[fi][fo][v]);
        }
      }
    }
    // A wave's 128 x 64 share is all inside the output or all past Na / Nb
    // (both multiples of 128, tile origins multiples of 256).  Lane (q, l16)
    // holds Out row wo + 16 fo + l16, In columns wi + 16 fi + 4q .. + 3.
    if (o0 + wo < Na && i0 + wi < Nb) {
      OT* og = out + (int64_t)g * Na * Nb;
      if constexpr (kPair) {
        // bf16 into a 16-byte aligned output: lanes of the row pair
        // (q, q ^ 1) trade halves of the instruction-tile pair (fi, fi + 1)
        // with one lane-row swap per value, so even q holds columns
        // 16 fi + 4q .. + 7 and odd q columns 16 fi + 4q + 12 .. + 19, and each
        // 16-byte store writes 64 contiguous bytes of an output row (the
        // 8-byte stores wrote 32, at the same count of write requests)
#pragma unroll
        for (int fo = 0; fo < 4; ++fo) {
#pragma unroll
          for (int fi = 0; fi < 8; fi += 2) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[fi][fo][e]),
                                                              __float_as_uint(acc[fi + 1][fo][e]), false, false);
              v[e] = __uint_as_float(r[0]);
              v[4 + e] = __uint_as_float(r[1]);
            }
            store8(og + (int64_t)(o0 + wo + 16 * fo + l16) * Nb + i0 + wi + 16 * fi + 4 * q + 12 * (q & 1), v,
                   kAcc);
          }
        }
      } else {
#pragma unroll
        for (int fo = 0; fo < 4; ++fo) {
#pragma unroll
          for (int fi = 0; fi < 8; ++fi) {
            const float v[4] = {acc[fi][fo][0], acc[fi][fo][1], acc[fi][fo][2], acc[fi][fo][3]};
            store4(og + (int64_t)(o0 + wo + 16 * fo + l16) * Nb + i0 + wi + 16 * fi + 4 * q, v, kAcc);
          }
        }
      }
    }
#pragma unroll
    for (int fi = 0; fi < 8; ++fi)
#pragma unroll
      for (int fo = 0; fo < 4; ++fo) acc[fi][fo] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_wgrad_padded_rows(int64_t M, int32_t G, int64_t* rows) {
  clear_detail();
  MOE_REQUIRE(rows, MOE_ERR_NULL, "rows is required");
  MOE_REQUIRE(M >= 0 && G >= 1, MOE_ERR_SHAPE, "M=%lld G=%d", (long long)M, G);
  MOE_REQUIRE(M <= kMaxElems, MOE_ERR_UNSUPPORTED, "M=%lld above 2^40", (long long)M);
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
  const int64_t blocks = ((M + 127) / 128 + G) * (int64_t)(C / 64);
  MOE_REQUIRE(blocks <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "too many (128-row tile, 64-column) blocks");
  hipStream_t s = as_stream(stream);
  padded_offsets_kernel<<<1, 256, 0, s>>>(group_offsets, G, padded_offsets);
  if (M > 0) {
    const dim3 grid((unsigned)blocks);
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
  MOE_REQUIRE(ld <= (int64_t(1) << 29), MOE_ERR_UNSUPPORTED, "ld=%lld above 2^29", (long long)ld);
  const int64_t n_tiles = (int64_t)G * ((Na + kWgTile - 1) / kWgTile) * ((Nb + kWgTile - 1) / kWgTile);
  MOE_REQUIRE(n_tiles <= 0x7fffffffLL - 8, MOE_ERR_UNSUPPORTED, "too many output tiles");
  MOE_REQUIRE(aq && as && bq && bs && padded_offsets && c, MOE_ERR_NULL, "every array is required");
  MOE_REQUIRE(aligned(aq, 16) && aligned(bq, 16) && aligned(as, 4) && aligned(bs, 4) &&
                  aligned(padded_offsets, 4) && aligned(c, c_dtype == MOE_F32 ? 16 : 8),
              MOE_ERR_ALIGN, "aq, bq (and a float32 c) need 16-byte alignment, a bf16 c 8-byte");
  hipStream_t s = as_stream(stream);
  // one workgroup per compute unit (its LDS ring fills one), each walking
  // its share of its XCD's tiles
  const int64_t per_xcd = (n_tiles + 7) / 8;
  int64_t nwg = (device_cu_count() + 7) / 8;
  if (nwg > per_xcd) nwg = per_xcd;
  const unsigned grid = (unsigned)(8 * nwg);
#define MOE_WGRAD_LAUNCH(OT, ACC, PAIR)                                                                     \
  wgrad_kernel<OT, ACC, PAIR><<<grid, kWgThreads, 0, s>>>(aq, as, bq, bs, padded_offsets, Na, Nb, ld, n_tiles, \
                                                          per_xcd, (int)nwg, static_cast<OT*>(c))
  if (c_dtype == MOE_F32) {
    if (accumulate) MOE_WGRAD_LAUNCH(float, true, false); else MOE_WGRAD_LAUNCH(float, false, false);
  } else if (aligned(c, 16)) {
    if (accumulate) MOE_WGRAD_LAUNCH(uint16_t, true, true); else MOE_WGRAD_LAUNCH(uint16_t, false, true);
  } else {
    if (accumulate) MOE_WGRAD_LAUNCH(uint16_t, true, false); else MOE_WGRAD_LAUNCH(uint16_t, false, false);
  }
#undef MOE_WGRAD_LAUNCH
  return after_launch("grouped_wgrad_fp8", s);
}
