// Block-scaled FP8 grouped GEMM for gfx950 ([DSV3-FP8]: FP8 expert GEMMs on
// 1x128 activation tiles and 128x128 weight blocks, with accumulation
// promoted to higher precision).
//
//   C[m, n] = sum_kb P_kb[m, n] * sa[m, kb] * sb_g[n / 128, kb]
//   P_kb    = FP8 dot product over the 128-wide K chunk kb (matrix cores)
//
// Design:
//  * The matrix core computes one whole 128-wide chunk per instruction
//    (V_MFMA_F32_16X16X128_F8F6F4, 16x16 outputs, zero C input), so its
//    float32 result is the chunk partial P_kb.  The promotion is one VALU
//    fused multiply-add per output per chunk: acc = fma(P_kb, sa * sb, acc),
//    in chunk order.
//  * Weight rows sit on the instruction's row axis and tokens on its column
//    axis: each lane's 4 outputs share one token (one sa per lane per chunk)
//    and 4 consecutive weight rows inside one 128-row block (one sb per wave
//    per chunk).
//  * Workgroup tile: 256 weight rows x 160 tokens of one group, 8 wavefronts
//    in a 4 (rows) x 2 (tokens) grid, each owning 64 x 80 outputs (4 x 5
//    instruction tiles, 80 float32 accumulators per lane).  160 tokens, not
//    128: a group slightly above the mean load (the usual case with top-K
//    routing) still fits one m-tile, so its weights are streamed once.
//  * Memory pipeline: a 3-stage LDS ring filled by direct global->LDS loads
//    (global_load_lds_dwordx4: no VGPR staging).  Each wave issues exactly
//    7 loads per K step (waves 0-3: 3 activation + 4 weight slices; waves
//    4-7: 2 activation + 4 weight slices + 1 scale load, which carries the
//    activation scales or, in wave 7, the two weight-block scales; past the
//    end the last chunk is re-fetched so the count never varies), so "chunk
//    kb has landed" is the wave's own s_waitcnt vmcnt(7) followed by a
//    barrier; two chunks (~106 KB) stay in flight per CU while one is
//    multiplied.  LDS rows are 128 bytes with a 16-byte XOR swizzle (applied
//    on the global side, since the DMA fixes lane -> LDS address), so the
//    32-byte operand reads spread over the banks.
//  * Optional row gather: row m of the grouped operand can be row a_row[m]
//    of aq / as (the permutation's token index), so the permuted copy of
//    the activations never has to be written; the indices only change the
//    per-lane load offsets of the activation slices and scales.
//  * Inner loop: per K chunk a wave's 4 x kTM instruction tiles run as one
//    straight-line software pipeline over its token tiles: token tile j's
//    four matrix products issue while the promotion FMAs of tile j - 1 run
//    on the vector ALU and tile j + 1's operand is read from LDS (the order
//    is pinned with scheduling-group barriers; left alone the compiler
//    issues all products first and all FMAs after, leaving the matrix core
//    idle during the FMAs, or hoists every read and runs out of registers).
//  * Ragged groups: token rows past the group's end are clamped on load and
//    never stored; a wave with no row of the group skips the chunk, the
//    others multiply all their instruction tiles (the clamped ones hold
//    copies of the last row and are discarded), so one body serves every
//    tile.
//  * Tile table on the device, no host sync: every workgroup reads the group
//    offsets, prefix-sums the m-tile counts in LDS (scratch aliased onto the
//    ring) and locates its own tile; the grid is sized from the host-known
//    bound floor(M / BM) + G m-tiles and surplus workgroups exit.
//  * XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
//    block b works on logical tile (b % 8) * ceil(tiles / 8) + b / 8.  Each
//    XCD sweeps a contiguous run of (group, n-tile, m-tile) tiles: the
//    m-tiles of one weight slab and the n-tiles of one activation tile run
//    together on one XCD and share its L2, so each weight byte crosses HBM
//    about once.
//  * Fused SwiGLU (grouped_gemm_fp8_swiglu): the weight tile is gate block c
//    (rows 128c..) stacked on up block c (rows I + 128c..); each wave holds
//    matching gate and up rows, so h = silu(g) * u forms in registers, the
//    1x128 amax of h along I is reduced across lanes and the 4 row-waves
//    through LDS, and only h's FP8 codes and scales are written.
#include "host_common.h"
#include "lds_dma.h"

#include <atomic>
#include <type_traits>

namespace moefp8 {
namespace {

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_SWIGLU = 2, OUT_COMBINE = 3 };

constexpr int kBN = 256;               // weight rows per workgroup tile (4 row-waves of 64)
constexpr int kMaxGroups = 1024;
constexpr int kMaxKB = 512;            // K <= 65536
constexpr int kMaxTilesPerWG = 64;     // tile-list entries per workgroup
constexpr int kMaxNTiles = 2048;       // n_tile field width of a tile-list entry
constexpr int kPersistentMaxKB = 32;   // persistent launch for K <= 4096

// Workgroup tile configuration: 256 weight rows x kBM tokens, 4 row-waves x
// kWMW token-waves, each wave 64 rows x kWM tokens (4 x kTM instruction
// tiles, 4 * kTM float32 accumulators per lane), a kStages-stage LDS ring.
// Every wave issues exactly kDma direct global->LDS loads per K step: kWOps
// weight slices, and kAHi activation slices (waves [0, kNHi)) or kAHi - 1
// activation slices plus one scale load (the other waves; scale load o
// carries the activation scales of tokens [64 o, 64 o + 64), the last one
// the two weight-block scales; waves beyond the needed count repeat a scale
// load, writing the same values to the same LDS words).
template <int kWMW_, int kTM_, int kStages_, int kAHi_, int kNHi_, int kMinBlocks_>
struct TileCfg {
  static constexpr int kWMW = kWMW_;
  static constexpr int kWaves = 4 * kWMW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kMinBlocks = kMinBlocks_;
  static constexpr int kTM = kTM_;
  static constexpr int kWM = 16 * kTM;
  static constexpr int kBM = kWMW * kWM;
  static constexpr int kStages = kStages_;
  static constexpr int kWOps = 32 / kWaves;
  static constexpr int kAHi = kAHi_;
  static constexpr int kNHi = kNHi_;
  static constexpr int kNScaleOps = (kBM + 63) / 64 + 1;
  static constexpr int kOffA = 0;                          // [kBM rows][128 B]
  static constexpr int kOffB = kBM * 128;                  // [256 rows][128 B]
  static constexpr int kOffS = kOffB + kBN * 128;          // activation scales, then weight-block scales
  static constexpr int kSB = 64 * (kNScaleOps - 1);        // float index of the weight-block scales
  static constexpr int kStageBytes = kOffS + kNScaleOps * 64 * 4;
  static constexpr int kDma = kWOps + kAHi;
  static constexpr int kGPT = kMaxGroups / kThreads;       // group-table entries per thread
  static_assert(kNHi * kAHi + (kWaves - kNHi) * (kAHi - 1) == kBM / 8, "activation slices");
  static_assert(kWaves - kNHi >= kNScaleOps, "scale loads");
  static_assert(kStages >= 2 && (kStages - 2) * kDma < 16, "wait count");
  static_assert(kStages * kStageBytes + kMaxTilesPerWG * 8 <= 160 * 1024, "LDS");
};
// 256 x 160, 8 waves, 3-stage ring (162816 B): a group a little above the
// mean top-K load still fits one m-tile, so its weight slab streams once.
using CfgS = TileCfg<2, 5, 3, 3, 4, 2>;

// One K chunk of a wave's tile for its first NA (active) 16-token
// instruction tiles, software-pipelined: the four chunk products of token
// tile j go to the matrix core while the promotion FMAs of tile j - 1 run on
// the vector ALU, and tile j + 1's operand is read from LDS meanwhile.  Each
// accumulator still receives one fma(P_kb, sa * sb, acc) per chunk, in chunk
// order.  tok: LDS rows of the wave's first token; sa_tok: their scales.
template <int NA, bool kFused, int kTM>
__device__ __forceinline__ void mma_chunk(v4f (&acc)[4][kTM], const v8i (&a_op)[4], const uint8_t* tok,
                                          const float* sa_tok, float sb0, float sb1, uint32_t lane_lo,
                                          uint32_t lane_hi, int l16) {
  v8i b_cur = lds_operand(tok, lane_lo, lane_hi);
  float sa_cur = sa_tok[l16];
  v4f p_prev[4];
  float sc0_prev = 0.f, sc1_prev = 0.f;
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    v8i b_next = b_cur;
    float sa_next = sa_cur;
    if (j + 1 < NA) {
      b_next = lds_operand(tok + 16 * (j + 1) * 128, lane_lo, lane_hi);
      sa_next = sa_tok[16 * (j + 1) + l16];
    }
    v4f p_cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p_cur[i] = mfma_chunk(a_op[i], b_cur);
    if (j > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = (kFused && i >= 2) ? sc1_prev : sc0_prev;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j - 1][v] = __builtin_fmaf(p_prev[i][v], sc, acc[i][j - 1][v]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) p_prev[i] = p_cur[i];
    sc0_prev = sa_cur * sb0;
    sc1_prev = kFused ? sa_cur * sb1 : sc0_prev;
    b_cur = b_next;
    sa_cur = sa_next;
    // order inside the stage: the next operand's LDS reads, then this tile's
    // four matrix products, then the previous tile's promotion FMAs (which
    // run while the products execute); keep the stages apart: hoisting every
    // tile's reads and products to the top would hold all their registers
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // matrix products
    __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);  // vector ALU
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sc = (kFused && i >= 2) ? sc1_prev : sc0_prev;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[i][NA - 1][v] = __builtin_fmaf(p_prev[i][v], sc, acc[i][NA - 1][v]);
  }
}

// The gate-weighted combine fused into the down projection's epilogue
// (OUT_COMBINE).  Each (token, n-tile) pair receives exactly topk grouped
// rows, one per selected expert, computed by topk workgroup tiles in any
// order.  A tile stores its float32 rows as usual, publishes them
// device-wide, and bumps one arrival counter per row; the tile that brings a
// counter to topk is the last one for that (token, n-tile), so every row it
// needs is already written.  It sums the token's topk rows over its 256
// columns in slot order, exactly as moe_combine does (the same binary32
// operations in the same order), adds the shared expert's row, and writes y
// in bf16.  The counter only elects who sums, never the order, so y is
// reproducible bit for bit; the elected tile resets the counter to zero.
struct CombineArgs {
  const int* row_token;  // [M] token of grouped row m
  const int* dst_row;    // [T, topk] grouped row of (token, slot)
  const float* gate;     // [T, topk]
  const float* shared;   // [T, N] or nullptr
  uint16_t* y;           // [T, N] bf16 bits
  int* counters;         // [T, n_tiles], zero between calls
  int T, topk;
  int64_t M;
};

// y[t, n_tile * 256 + 4 lane .. + 4] of one elected token (one wavefront).
__device__ __forceinline__ void combine_token(const CombineArgs& cb, const float* c, int t, int col, int N) {
  constexpr int kBatch = 8;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int* drow = cb.dst_row + (int64_t)t * cb.topk;
  const float* grow = cb.gate + (int64_t)t * cb.topk;
  for (int k0 = 0; k0 < cb.topk; k0 += kBatch) {
    u32x4 v[kBatch];
    float g[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + j < cb.topk) {
        const int r = min(max(drow[k0 + j], 0), (int)cb.M - 1);
        g[j] = grow[k0 + j];
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c + (int64_t)r * N + col));
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + j < cb.topk) {
        acc[0] = acc[0] + g[j] * __uint_as_float(v[j][0]);
        acc[1] = acc[1] + g[j] * __uint_as_float(v[j][1]);
        acc[2] = acc[2] + g[j] * __uint_as_float(v[j][2]);
        acc[3] = acc[3] + g[j] * __uint_as_float(v[j][3]);
      }
    }
  }
  if (cb.shared) {
    const u32x4 s4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cb.shared + (int64_t)t * N + col));
    acc[0] = acc[0] + __uint_as_float(s4[0]);
    acc[1] = acc[1] + __uint_as_float(s4[1]);
    acc[2] = acc[2] + __uint_as_float(s4[2]);
    acc[3] = acc[3] + __uint_as_float(s4[3]);
  }
  uint2 o;
  o.x = bf16_rne_bits(acc[0]) | (bf16_rne_bits(acc[1]) << 16);
  o.y = bf16_rne_bits(acc[2]) | (bf16_rne_bits(acc[3]) << 16);
  *reinterpret_cast<uint2*>(cb.y + (int64_t)t * N + col) = o;
}

// Called by every wave after the tile's rows are stored; `lds` is the ring
// stage just multiplied (free until the next K step's barrier).  One
// device-scope release and one acquire per tile, both in wave 0: every wave
// first waits for its own stores, the workgroup barrier orders them before
// wave 0's release, and the second barrier orders wave 0's acquire before
// the other waves' loads.
template <class C>
__device__ __forceinline__ void combine_epilogue(const CombineArgs& cb, uint8_t* lds, const float* c, int row0,
                                                 int rows_valid, int n_tile, int n_tiles, int N) {
  constexpr int kRW = (C::kBM + 63) / 64;  // 64-row groups of the tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int* sTok = reinterpret_cast<int*>(lds);  // [kRW][64] elected tokens
  int* sCnt = sTok + kRW * 64;              // [kRW]
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's rows are written
  __syncthreads();                           // ... every wave's; the stage is free
  if (w == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // publish the tile's rows device-wide
    uint64_t any = 0;
#pragma unroll
    for (int rw = 0; rw < kRW; ++rw) {
      const int r = rw * 64 + lane;
      int t = 0;
      bool last = false;
      if (r < rows_valid) {
        t = cb.row_token[row0 + r];
        if ((unsigned)t < (unsigned)cb.T) {
          int* ctr = cb.counters + (int64_t)t * n_tiles + n_tile;
          last = atomicAdd(ctr, 1) == cb.topk - 1;
          if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const uint64_t m = __ballot(last);
      if (last) sTok[rw * 64 + __popcll(m & ((1ull << lane) - 1ull))] = t;
      if (lane == 0) sCnt[rw] = __popcll(m);
      any |= m;
    }
    if (any) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other tiles' rows
  }
  __syncthreads();
  const int col = n_tile * kBN + 4 * lane;
  int j = 0;
#pragma unroll
  for (int rw = 0; rw < kRW; ++rw) {
    const int cnt = __builtin_amdgcn_readfirstlane(sCnt[rw]);
    for (int i = 0; i < cnt; ++i, ++j) {
      if (j % C::kWaves != w) continue;
      const int t = __builtin_amdgcn_readfirstlane(sTok[rw * 64 + i]);
      if (col < N) combine_token(cb, c, t, col, N);
    }
  }
}

template <int MODE, class C>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void grouped_gemm_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ as, const int* __restrict__ a_row, int a_rows,
    const uint8_t* __restrict__ bq, const float* __restrict__ bs, const int* __restrict__ offsets, int G,
    int N, int K, int n_tiles, int wg_per_xcd, void* __restrict__ out, float* __restrict__ hs_out,
    CombineArgs cmb) {
  constexpr bool kFused = MODE == OUT_SWIGLU;
  constexpr int kThreads = C::kThreads, kBM = C::kBM, kWM = C::kWM, kTM = C::kTM, kStages = C::kStages;
  constexpr int kStageBytes = C::kStageBytes, kOffA = C::kOffA, kOffB = C::kOffB, kOffS = C::kOffS;
  constexpr int kSB = C::kSB, kWOps = C::kWOps, kAHi = C::kAHi, kNHi = C::kNHi, kGPT = C::kGPT;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kStageBytes];
  __shared__ int2 sTile[kMaxTilesPerWG];  // {g | n_tile << 10 | rows_valid << 21, row0}

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) wave index
  const int wn = w & 3, wm = w >> 2;
  const int q = lane >> 4, l16 = lane & 15;
  const int KB = K / 128;
  const int I = N / 2;  // fused: gate rows [0, I), up rows [I, 2I)
  const int nblk = N / 128;

  // ---- this workgroup's tile list (group table scratch aliased onto the ring) ----
  int n_my;
  {
    int* sP = reinterpret_cast<int*>(ring);  // [G + 1] m-tile prefix
    int* sOff = sP + (kMaxGroups + 1);       // [G + 1] row offsets
    int* sScan = sOff + (kMaxGroups + 1);    // [kThreads]
    int mt[kGPT];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kGPT; ++i) {
      const int g = tid * kGPT + i;
      mt[i] = 0;
      if (g < G) {
        const int o0 = offsets[g], o1 = offsets[g + 1];
        sOff[g] = o0;
        mt[i] = (o1 - o0 + kBM - 1) / kBM;
        if (g == G - 1) sOff[G] = o1;
      }
      local += mt[i];
    }
    sScan[tid] = local;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
      const int v = tid >= d ? sScan[tid - d] : 0;
      __syncthreads();
      sScan[tid] += v;
      __syncthreads();
    }
    int run = sScan[tid] - local;
#pragma unroll
    for (int i = 0; i < kGPT; ++i) {
      const int g = tid * kGPT + i;
      if (g < G) sP[g] = run;
      run += mt[i];
    }
    if (tid == kThreads - 1) sP[G] = sScan[kThreads - 1];
    __syncthreads();
    // XCD x sweeps logical tiles [x * per_xcd, (x + 1) * per_xcd); its
    // workgroup s takes every wg_per_xcd-th of them, starting at s
    const int total = sP[G] * n_tiles;
    const int per_xcd = (total + 7) / 8;
    const int lo = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int hi = min(total, (int)(blockIdx.x & 7) * per_xcd + per_xcd);
    n_my = lo < hi ? min((hi - lo + wg_per_xcd - 1) / wg_per_xcd, kMaxTilesPerWG) : 0;
    if (tid < n_my) {
      const int lid = lo + tid * wg_per_xcd;
      int lo_g = 0, hi_g = G;
      while (lo_g < hi_g) {
        const int mid = (lo_g + hi_g + 1) >> 1;
        if (sP[mid] * n_tiles <= lid) lo_g = mid; else hi_g = mid - 1;
      }
      const int g = lo_g;
      const int mt_g = sP[g + 1] - sP[g];
      const int local_id = lid - sP[g] * n_tiles;
      const int n_tile = local_id / mt_g;
      const int row0 = sOff[g] + (local_id % mt_g) * kBM;
      const int rows_valid = min(kBM, sOff[g + 1] - row0);
      sTile[tid] = make_int2(g | (n_tile << 10) | (rows_valid << 21), row0);
    }
    __syncthreads();  // tile list visible; the ring is free again
  }
  if (n_my == 0) return;

  // ---- issue side: one continuous chunk stream over all of this workgroup's tiles ----
  const int p16 = lane & 7;   // physical 16-byte piece inside the LDS row
  const int rsub = lane >> 3;  // row inside the 8-row (1 KB) DMA slice
  const int c16 = p16 ^ rsub;  // logical piece it must fetch (swizzle)
  // activation slices (8 rows each): waves [0, kNHi) take kAHi, the others
  // kAHi - 1 and one scale load (see TileCfg)
  const bool a_hi = w < kNHi;
  const int a_slice0 = a_hi ? kAHi * w : kAHi * kNHi + (kAHi - 1) * (w - kNHi);
  const int s_op = a_hi ? 0 : (w - kNHi) % C::kNScaleOps;  // scale load of this wave
  const bool s_weight = s_op == C::kNScaleOps - 1;          // ... the weight-block scales
  const uint8_t* ia_base = aq;  // scalar bases of the tile being issued
  const uint8_t* ib_base = bq;
  const uint8_t* is_base = reinterpret_cast<const uint8_t*>(as);
  uint32_t ia_off[kAHi], ib_off[kWOps], is_off = 0;  // per-lane byte offsets from them
  int it = 0, ikb = 0;                                // next chunk to issue: tile it, chunk ikb
  auto load_issue_tile = [&](int i) {
    const int2 e = sTile[i];
    const int wd = __builtin_amdgcn_readfirstlane(e.x);
    const int row0 = __builtin_amdgcn_readfirstlane(e.y);
    const int g = wd & 1023, n_tile = (wd >> 10) & 2047, rows_valid = wd >> 21;
    // activation rows: row0 + r of the grouped operand, or aq[a_row[row0 + r]]
    // when gathering (indices clamped into [0, a_rows); the host bounds
    // a_rows * K by 2^32 so the 32-bit offsets hold)
    if (a_row != nullptr) {
      ia_base = aq;
#pragma unroll
      for (int j = 0; j < kAHi; ++j) {
        const int src = min(max(a_row[row0 + min((a_slice0 + j) * 8 + rsub, rows_valid - 1)], 0), a_rows - 1);
        ia_off[j] = (uint32_t)src * (uint32_t)K + (uint32_t)(c16 * 16);
      }
    } else {
      ia_base = aq + (int64_t)row0 * K;
#pragma unroll
      for (int j = 0; j < kAHi; ++j)
        ia_off[j] = (uint32_t)(min((a_slice0 + j) * 8 + rsub, rows_valid - 1) * K + c16 * 16);
    }
    const uint8_t* bq_g = bq + (int64_t)g * N * K;
    if (kFused) {
      // weight slices 0..15 hold gate block n_tile, 16..31 the matching up
      // block; a wave's slices lie in one half
      const int half = (w * kWOps) / 16;
      ib_base = bq_g + (int64_t)((half ? I : 0) + n_tile * 128) * K;
#pragma unroll
      for (int j = 0; j < kWOps; ++j) ib_off[j] = (uint32_t)((((w * kWOps + j) % 16) * 8 + rsub) * K + c16 * 16);
    } else {
      ib_base = bq_g + (int64_t)n_tile * kBN * K;
      const int last = N - 1 - n_tile * kBN;  // rows past N (a half tile) re-read row N - 1
#pragma unroll
      for (int j = 0; j < kWOps; ++j) ib_off[j] = (uint32_t)(min((w * kWOps + j) * 8 + rsub, last) * K + c16 * 16);
    }
    if (a_hi) {
      // no scale load
    } else if (!s_weight) {
      const int t = min(s_op * 64 + lane, rows_valid - 1);
      if (a_row != nullptr) {
        is_base = reinterpret_cast<const uint8_t*>(as);
        is_off = (uint32_t)min(max(a_row[row0 + t], 0), a_rows - 1) * (uint32_t)(KB * 4);
      } else {
        is_base = reinterpret_cast<const uint8_t*>(as + (int64_t)row0 * KB);
        is_off = (uint32_t)(t * KB * 4);
      }
    } else {
      const int blkA = kFused ? n_tile : 2 * n_tile;
      const int blkB = kFused ? I / 128 + n_tile : min(2 * n_tile + 1, nblk - 1);
      is_base = reinterpret_cast<const uint8_t*>(bs + ((int64_t)g * nblk + blkA) * KB);
      is_off = (uint32_t)(lane == 0 ? 0 : (blkB - blkA) * KB * 4);
    }
  };
  // Enqueue chunk (it, ikb) into the stage at LDS address `st`, then advance;
  // past the last chunk the last chunk is re-fetched, so every call issues
  // exactly kDma loads per wave.
  auto issue_next = [&](uint32_t st) {
    const uint8_t* a = ia_base + ikb * 128;
    const uint8_t* b = ib_base + ikb * 128;
#pragma unroll
    for (int j = 0; j < kAHi - 1; ++j) dma16(a, ia_off[j], st + kOffA + (a_slice0 + j) * 1024);
    if (a_hi) dma16(a, ia_off[kAHi - 1], st + kOffA + (a_slice0 + kAHi - 1) * 1024);
    else dma4(is_base + ikb * 4, is_off, st + kOffS + s_op * 256);
#pragma unroll
    for (int j = 0; j < kWOps; ++j) dma16(b, ib_off[j], st + kOffB + (w * kWOps + j) * 1024);
    if (ikb + 1 < KB) {
      ++ikb;
    } else if (it + 1 < n_my) {
      ++it;
      ikb = 0;
      load_issue_tile(it);
    }
  };

  // ---- wave geometry ----
  const uint32_t lane_lo = frag_lane_lo(lane);
  const uint32_t lane_hi = lane_lo ^ 16;
  // first weight row of instruction tile i (rows 16 i' + lane % 16)
  auto brow0 = [&](int i) { return kFused ? (i < 2 ? 0 : 128) + 32 * wn + 16 * (i & 1) : 64 * wn + 16 * i; };
  const int sb_sel = kFused ? 0 : (wn >> 1);  // unfused: rows of row-waves 0,1 in block A, 2,3 in B

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  load_issue_tile(0);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue_next(ring_lds + s * kStageBytes);
  int ist = kStages - 1, cst = 0;  // stage receiving the next issue / holding the next chunk to multiply

  for (int ti = 0; ti < n_my; ++ti) {
    const int2 e = sTile[ti];
    const int wd = __builtin_amdgcn_readfirstlane(e.x);
    const int row0 = __builtin_amdgcn_readfirstlane(e.y);
    const int n_tile = (wd >> 10) & 2047, rows_valid = wd >> 21;
    int n_active = 0;
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      if (wm * kWM + 16 * j < rows_valid) n_active = j + 1;
    if (!kFused && n_tile * kBN + wn * 64 >= N) n_active = 0;  // half tile: rows past N

    v4f acc[4][kTM];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const uint8_t* st = ring;
    for (int kb = 0; kb < KB; ++kb) {
      // this wave's loads of the chunk in stage cst have landed (only the
      // later chunks' may still fly; loads complete in issue order) ...
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * C::kDma));
      // ... and every other wave's too; all waves are also done with the
      // previous chunk, whose stage receives the chunk kStages - 1 ahead now
      __builtin_amdgcn_s_barrier();
      issue_next(ring_lds + ist * kStageBytes);
      ist = ist == kStages - 1 ? 0 : ist + 1;
      st = ring + cst * kStageBytes;
      cst = cst == kStages - 1 ? 0 : cst + 1;

      const float* sS = reinterpret_cast<const float*>(st + kOffS);
      v8i a_op[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a_op[i] = lds_operand(st + kOffB + brow0(i) * 128, lane_lo, lane_hi);
      const float sb0 = kFused ? sS[kSB] : sS[kSB + sb_sel];
      const float sb1 = kFused ? sS[kSB + 1] : sb0;
      // every instruction tile of the wave, active or not (a ragged tile's
      // inactive ones hold clamped copies of its last row and are never
      // stored): one straight-line, software-pipelined body
      if (n_active > 0)
        mma_chunk<kTM, kFused, kTM>(acc, a_op, st + kOffA + wm * kWM * 128, sS + wm * kWM, sb0, sb1, lane_lo,
                                    lane_hi, l16);
    }

    // ---- epilogue (the next tile's first chunks keep streaming in) ----
    if constexpr (!kFused) {
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        const int mloc = wm * kWM + 16 * j + l16;
        if (j < n_active && mloc < rows_valid) {
          const int64_t m = row0 + mloc;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = n_tile * kBN + wn * 64 + 16 * i + 4 * q;
            if (MODE == OUT_F32 || MODE == OUT_COMBINE) {
              float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + m * N + n) = v;
            } else {
              uint2 v;
              v.x = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
              v.y = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + m * N + n) = v;
            }
          }
        }
      }
      if constexpr (MODE == OUT_COMBINE)
        combine_epilogue<C>(cmb, const_cast<uint8_t*>(st), reinterpret_cast<const float*>(out), row0, rows_valid,
                            n_tile, n_tiles, N);
    } else {
      // h = silu(g) * u into the gate accumulators; per-token amax over this
      // wave's 32 h columns, then across the 4 row-waves through LDS.  The
      // exchange uses the stage just multiplied: it is not refilled before
      // the next K step's barrier.
      float(*sAmax)[kBM] = reinterpret_cast<float(*)[kBM]>(const_cast<uint8_t*>(st));
      lds_barrier();  // every wave is done reading that stage
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float h = spec_silu(acc[i][j][v]) * acc[i + 2][j][v];
            acc[i][j][v] = h;
            amax = fmaxf(amax, fabsf(h));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (q == 0) sAmax[wn][wm * kWM + 16 * j + l16] = amax;
      }
      lds_barrier();  // partial maxima visible
      uint8_t* hq = reinterpret_cast<uint8_t*>(out);
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        const int mloc = wm * kWM + 16 * j + l16;
        if (j < n_active && mloc < rows_valid) {
          const float amax = fmaxf(fmaxf(sAmax[0][mloc], sAmax[1][mloc]), fmaxf(sAmax[2][mloc], sAmax[3][mloc]));
          const float sc = scale_from_amax(amax);
          const Divider div(sc);
          const int64_t m = row0 + mloc;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int col = n_tile * 128 + 32 * wn + 16 * i + 4 * q;
            const uint32_t wd4 = quantize4(div, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint32_t*>(hq + m * I + col) = wd4;
          }
          if (wn == 0 && q == 0) hs_out[m * (I / 128) + n_tile] = sc;
        }
      }
    }
  }
  // the trailing re-fetches must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}


template <int MODE, class C>
moe_status launch_cfg(const uint8_t* aq, const float* as, const int* a_row, int64_t a_rows, const uint8_t* bq,
                      const float* bs, const int* offsets, int G, int64_t M, int N, int K, int n_tiles, void* out,
                      float* hs, const CombineArgs& cmb, hipStream_t st, const char* what) {
  // Upper bound on the m-tiles: sum_g ceil(M_g / BM) <= floor(M / BM) + G, and
  // every m-tile holds at least one row.
  int64_t mt_bound = M / C::kBM + G;
  if (mt_bound > M) mt_bound = M;
  const int64_t tiles = mt_bound * n_tiles;
  if (tiles == 0) return MOE_OK;
  if (tiles >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", what);
  // Short tiles (K <= 128 kPersistentMaxKB): one resident workgroup per
  // compute unit (the LDS ring fills a CU) walks a list of tiles with the
  // ring running across tile boundaries, which hides the per-tile pipeline
  // fill, table build and epilogue; at most kMaxTilesPerWG tiles each.  Long
  // tiles: one tile per workgroup, so the dispatcher balances the tail.
  const int64_t per_xcd = (tiles + 7) / 8;
  int64_t wg_per_xcd = per_xcd;
  if (K / 128 <= kPersistentMaxKB) {
    wg_per_xcd = (device_cu_count() + 7) / 8;
    const int64_t need = (per_xcd + kMaxTilesPerWG - 1) / kMaxTilesPerWG;
    if (wg_per_xcd < need) wg_per_xcd = need;
    if (wg_per_xcd > per_xcd) wg_per_xcd = per_xcd;
  }
  // every workgroup's share of its XCD's tiles fits its tile list (the
  // kernel would otherwise drop the excess)
  if ((per_xcd + wg_per_xcd - 1) / wg_per_xcd > kMaxTilesPerWG)
    return fail(MOE_ERR_UNSUPPORTED, "%s: tile list overflow", what);
  grouped_gemm_kernel<MODE, C><<<(unsigned)(8 * wg_per_xcd), C::kThreads, 0, st>>>(
      aq, as, a_row, (int)a_rows, bq, bs, offsets, G, N, K, n_tiles, (int)wg_per_xcd, out, hs, cmb);
  return after_launch(what, st);
}

template <int MODE>
moe_status launch_gemm(const uint8_t* aq, const float* as, const int* a_row, int64_t a_rows,
                       const uint8_t* bq, const float* bs, const int* offsets, int G, int64_t M, int N,
                       int K, void* out, float* hs, hipStream_t st, const char* what,
                       const CombineArgs& cmb = CombineArgs{}) {
  const int n_tiles = (int)(MODE == OUT_SWIGLU ? (N / 2) / 128 : ((int64_t)N + kBN - 1) / kBN);
  if (n_tiles > kMaxNTiles) return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d too large", what, N);
  return launch_cfg<MODE, CfgS>(aq, as, a_row, a_rows, bq, bs, offsets, G, M, N, K, n_tiles, out, hs, cmb, st,
                                what);
}

moe_status check_gemm_args(const uint8_t* aq, const float* as, const int32_t* a_row, int64_t a_rows,
                           const uint8_t* bq, const float* bs, const int32_t* offsets, int32_t G,
                           int64_t M, int32_t N, int32_t K) {
  MOE_REQUIRE(G >= 1 && M >= 0 && N > 0 && K > 0, MOE_ERR_SHAPE, "G=%d M=%lld N=%d K=%d", G,
              (long long)M, N, K);
  MOE_REQUIRE(G <= kMaxGroups, MOE_ERR_UNSUPPORTED, "G=%d > %d", G, kMaxGroups);
  MOE_REQUIRE(N % 128 == 0 && K % 128 == 0, MOE_ERR_SHAPE, "N=%d and K=%d must be multiples of 128", N, K);
  MOE_REQUIRE(K <= 128 * kMaxKB, MOE_ERR_UNSUPPORTED, "K=%d > %d", K, 128 * kMaxKB);
  MOE_REQUIRE(M < (1LL << 31), MOE_ERR_UNSUPPORTED, "M too large");
  MOE_REQUIRE(offsets, MOE_ERR_NULL, "group_offsets is required");
  MOE_REQUIRE(aligned(offsets, 4), MOE_ERR_ALIGN, "group_offsets needs 4-byte alignment");
  if (M == 0) return MOE_OK;
  MOE_REQUIRE(aq && as && bq && bs, MOE_ERR_NULL, "aq, as, bq and bs are required");
  MOE_REQUIRE(aligned(aq, 16) && aligned(bq, 16) && aligned(as, 4) && aligned(bs, 4), MOE_ERR_ALIGN,
              "aq and bq need 16-byte alignment, scales 4-byte");
  if (a_row) {
    MOE_REQUIRE(aligned(a_row, 4), MOE_ERR_ALIGN, "a_row needs 4-byte alignment");
    MOE_REQUIRE(a_rows >= 1, MOE_ERR_SHAPE, "a_rows=%lld must be positive with a_row", (long long)a_rows);
    MOE_REQUIRE(a_rows * (int64_t)K <= (1LL << 32), MOE_ERR_UNSUPPORTED,
                "gathered operand of %lld x %d bytes exceeds 4 GiB", (long long)a_rows, K);
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

namespace moefp8 {
namespace {

moe_status gemm_entry(const uint8_t* aq, const float* as, const int32_t* a_row, int64_t a_rows,
                      const uint8_t* bq, const float* bs, const int32_t* group_offsets, int32_t G, int64_t M,
                      int32_t N, int32_t K, void* c, moe_dtype c_dtype, void* stream, const char* what) {
  MOE_REQUIRE(c_dtype == MOE_F32 || c_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "c_dtype %d", (int)c_dtype);
  moe_status stt = check_gemm_args(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(c, MOE_ERR_NULL, "c is required");
  MOE_REQUIRE(aligned(c, 16), MOE_ERR_ALIGN, "c needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  if (c_dtype == MOE_F32)
    return launch_gemm<OUT_F32>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K, c, nullptr, st, what);
  return launch_gemm<OUT_BF16>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K, c, nullptr, st, what);
}

}  // namespace
}  // namespace moefp8

extern "C" moe_status grouped_gemm_fp8_blockscaled(const uint8_t* aq, const float* as, const uint8_t* bq,
                                                   const float* bs, const int32_t* group_offsets, int32_t G,
                                                   int64_t M, int32_t N, int32_t K, void* c, moe_dtype c_dtype,
                                                   void* stream) {
  clear_detail();
  return gemm_entry(aq, as, nullptr, 0, bq, bs, group_offsets, G, M, N, K, c, c_dtype, stream,
                    "grouped_gemm_fp8_blockscaled");
}

extern "C" moe_status grouped_gemm_fp8_blockscaled_gather(const uint8_t* aq, const float* as,
                                                          const int32_t* a_row, int64_t a_rows,
                                                          const uint8_t* bq, const float* bs,
                                                          const int32_t* group_offsets, int32_t G, int64_t M,
                                                          int32_t N, int32_t K, void* c, moe_dtype c_dtype,
                                                          void* stream) {
  clear_detail();
  MOE_REQUIRE(a_row != nullptr || M == 0, MOE_ERR_NULL, "a_row is required");
  return gemm_entry(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K, c, c_dtype, stream,
                    "grouped_gemm_fp8_blockscaled_gather");
}

extern "C" moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, const int32_t* a_row,
                                              int64_t a_rows, const uint8_t* bq, const float* bs,
                                              const int32_t* group_offsets, int32_t G, int64_t M,
                                              int32_t I, int32_t K, uint8_t* hq, float* hs,
                                              void* stream) {
  clear_detail();
  MOE_REQUIRE(I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "I=%d must be a positive multiple of 128", I);
  MOE_REQUIRE(I <= 128 * kMaxNTiles, MOE_ERR_UNSUPPORTED, "I=%d > %d", I, 128 * kMaxNTiles);
  moe_status stt = check_gemm_args(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, 2 * I, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(hq && hs, MOE_ERR_NULL, "hq and hs are required");
  MOE_REQUIRE(aligned(hq, 16) && aligned(hs, 4), MOE_ERR_ALIGN, "hq needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  return launch_gemm<OUT_SWIGLU>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, 2 * I, K, hq, hs, st,
                                 "grouped_gemm_fp8_swiglu");
}

extern "C" moe_status grouped_gemm_fp8_combine_workspace_size(int32_t T, int32_t N, size_t* bytes) {
  clear_detail();
  MOE_REQUIRE(bytes, MOE_ERR_NULL, "bytes is required");
  MOE_REQUIRE(T >= 0 && N > 0, MOE_ERR_SHAPE, "T=%d N=%d", T, N);
  *bytes = (size_t)T * (((size_t)N + kBN - 1) / kBN) * sizeof(int32_t);
  return MOE_OK;
}

extern "C" moe_status grouped_gemm_fp8_combine(const uint8_t* aq, const float* as, const uint8_t* bq,
                                               const float* bs, const int32_t* group_offsets, int32_t G, int64_t M,
                                               int32_t N, int32_t K, float* c, const int32_t* src_token,
                                               const int32_t* dst_row, const float* topk_gate, const float* shared,
                                               int32_t T, int32_t topk, uint16_t* y_bf16, int32_t* counters,
                                               size_t counters_bytes, void* stream) {
  clear_detail();
  MOE_REQUIRE(T >= 0 && topk >= 1, MOE_ERR_SHAPE, "T=%d topk=%d", T, topk);
  MOE_REQUIRE(M == (int64_t)T * topk, MOE_ERR_SHAPE, "M=%lld must equal T*topk=%lld (no token dropped)",
              (long long)M, (long long)T * topk);
  moe_status stt = check_gemm_args(aq, as, nullptr, 0, bq, bs, group_offsets, G, M, N, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(c && src_token && dst_row && topk_gate && y_bf16 && counters, MOE_ERR_NULL,
              "c, src_token, dst_row, topk_gate, y and counters are required");
  MOE_REQUIRE(aligned(c, 16) && aligned(shared, 16) && aligned(y_bf16, 16) && aligned(src_token, 4) &&
                  aligned(dst_row, 4) && aligned(topk_gate, 4) && aligned(counters, 4),
              MOE_ERR_ALIGN, "c, shared and y need 16-byte alignment, index arrays 4-byte");
  size_t need = 0;
  grouped_gemm_fp8_combine_workspace_size(T, N, &need);
  MOE_REQUIRE(counters_bytes >= need, MOE_ERR_WORKSPACE, "counters %zu < %zu bytes", counters_bytes, need);
  CombineArgs cb;
  cb.row_token = src_token;
  cb.dst_row = dst_row;
  cb.gate = topk_gate;
  cb.shared = shared;
  cb.y = y_bf16;
  cb.counters = counters;
  cb.T = T;
  cb.topk = topk;
  cb.M = M;
  return launch_gemm<OUT_COMBINE>(aq, as, nullptr, 0, bq, bs, group_offsets, G, M, N, K, c, nullptr,
                                  as_stream(stream), "grouped_gemm_fp8_combine", cb);
}
