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
//  * Ragged groups: token rows past the group's end are clamped on load and
//    never stored; 16-row instruction tiles past the end are skipped, so a
//    group of M_g rows costs ceil(M_g / 16) tiles of matrix work.
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

#include <type_traits>

namespace moefp8 {
namespace {

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_SWIGLU = 2 };

constexpr int kThreads = 512;          // 8 wavefronts
constexpr int kBN = 256;               // weight rows per workgroup tile
constexpr int kBM = 160;               // tokens per workgroup tile
constexpr int kWM = kBM / 2;           // tokens per wavefront
constexpr int kTM = kWM / 16;          // 16-token instruction tiles per wavefront
constexpr int kStages = 3;
constexpr int kMaxGroups = 1024;
constexpr int kMaxKB = 512;            // K <= 65536
constexpr int kOffA = 0;                         // [160 rows][128 B]
constexpr int kOffB = kBM * 128;                 // [256 rows][128 B]
constexpr int kOffS = kOffB + kBN * 128;         // [256] float: 192 activation scales, 2 weight scales
constexpr int kSB = 192;                         // float index of the weight-block scales in S
constexpr int kStageBytes = kOffS + 4 * 64 * 4;  // 54272; 3 stages = 162816 B of LDS
constexpr int kDmaPerChunk = 7;                  // per wave, see the memory pipeline notes
constexpr int kMaxTilesPerWG = 64;              // tile-list entries per workgroup
constexpr int kMaxNTiles = 2048;                 // n_tile field width of a tile-list entry
constexpr int kPersistentMaxKB = 32;             // persistent launch for K <= 4096

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ as, const int* __restrict__ a_row, int a_rows,
    const uint8_t* __restrict__ bq, const float* __restrict__ bs, const int* __restrict__ offsets, int G,
    int N, int K, int n_tiles, int wg_per_xcd, void* __restrict__ out, float* __restrict__ hs_out) {
  constexpr bool kFused = MODE == OUT_SWIGLU;
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
    int mt[2];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = tid * 2 + i;
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
    for (int i = 0; i < 2; ++i) {
      const int g = tid * 2 + i;
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
  // activation slices (8 rows each): waves 0-3 take 3, waves 4-7 take 2; the
  // scale load of waves 4-7 fills S: S[t] = sa of token t (t < 192, rows
  // past the group clamped), S[192] / S[193] = weight-block scales A / B
  const bool a3 = w < 4;
  const int a_slice0 = a3 ? 3 * w : 12 + 2 * (w - 4);
  const uint8_t* ia_base = aq;  // scalar bases of the tile being issued
  const uint8_t* ib_base = bq;
  const uint8_t* is_base = reinterpret_cast<const uint8_t*>(as);
  uint32_t ia_off[3], ib_off[4], is_off = 0;  // per-lane byte offsets from them
  int it = 0, ikb = 0;                         // next chunk to issue: tile it, chunk ikb
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
      for (int j = 0; j < 3; ++j) {
        const int src = min(max(a_row[row0 + min((a_slice0 + j) * 8 + rsub, rows_valid - 1)], 0), a_rows - 1);
        ia_off[j] = (uint32_t)src * (uint32_t)K + (uint32_t)(c16 * 16);
      }
    } else {
      ia_base = aq + (int64_t)row0 * K;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        ia_off[j] = (uint32_t)(min((a_slice0 + j) * 8 + rsub, rows_valid - 1) * K + c16 * 16);
    }
    const uint8_t* bq_g = bq + (int64_t)g * N * K;
    if (kFused) {
      // waves 0-3 fetch gate block n_tile, waves 4-7 the matching up block
      ib_base = bq_g + (int64_t)((w < 4 ? 0 : I) + n_tile * 128) * K;
#pragma unroll
      for (int j = 0; j < 4; ++j) ib_off[j] = (uint32_t)((((w & 3) * 4 + j) * 8 + rsub) * K + c16 * 16);
    } else {
      ib_base = bq_g + (int64_t)n_tile * kBN * K;
      const int last = N - 1 - n_tile * kBN;  // rows past N (a half tile) re-read row N - 1
#pragma unroll
      for (int j = 0; j < 4; ++j) ib_off[j] = (uint32_t)(min((w * 4 + j) * 8 + rsub, last) * K + c16 * 16);
    }
    if (w < 4) {
      // no scale load
    } else if (w < 7) {
      const int t = min((w - 4) * 64 + lane, rows_valid - 1);
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
  // exactly kDmaPerChunk loads per wave.
  auto issue_next = [&](uint32_t st) {
    const uint8_t* a = ia_base + ikb * 128;
    const uint8_t* b = ib_base + ikb * 128;
    dma16(a, ia_off[0], st + kOffA + a_slice0 * 1024);
    dma16(a, ia_off[1], st + kOffA + (a_slice0 + 1) * 1024);
    if (a3) dma16(a, ia_off[2], st + kOffA + (a_slice0 + 2) * 1024);
    else dma4(is_base + ikb * 4, is_off, st + kOffS + (w - 4) * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(b, ib_off[j], st + kOffB + (w * 4 + j) * 1024);
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
  const int sb_sel = kFused ? 0 : (wn >> 1);  // unfused: rows of waves 0,1 in block A, 2,3 in B

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  load_issue_tile(0);
  issue_next(ring_lds);
  issue_next(ring_lds + kStageBytes);
  int ist = 2, cst = 0;  // stage receiving the next issue / holding the next chunk to multiply

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
      // this wave's loads of the chunk in stage cst have landed (only the next
      // chunk's may still fly; loads complete in issue order) ...
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerChunk));
      // ... and every other wave's too; all waves are also done with the
      // previous chunk, whose stage receives the chunk after next now
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
      // active tiles are a prefix (j < n_active): leaving at the first
      // inactive one gives the compiler one nested region to schedule
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        if (j >= n_active) break;
        const v8i b_op = lds_operand(st + kOffA + (wm * kWM + 16 * j) * 128, lane_lo, lane_hi);
        const float sa = sS[wm * kWM + 16 * j + l16];
        const float sc0 = sa * sb0;
        const float sc1 = kFused ? sa * sb1 : sc0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4f p = mfma_chunk(a_op[i], b_op);
          const float sc = (kFused && i >= 2) ? sc1 : sc0;
          acc[i][j][0] = __builtin_fmaf(p[0], sc, acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(p[1], sc, acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(p[2], sc, acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(p[3], sc, acc[i][j][3]);
        }
      }
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
            if (MODE == OUT_F32) {
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

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int MODE>
moe_status launch_gemm(const uint8_t* aq, const float* as, const int* a_row, int64_t a_rows,
                       const uint8_t* bq, const float* bs, const int* offsets, int G, int64_t M, int N,
                       int K, void* out, float* hs, hipStream_t st, const char* what) {
  const int n_tiles = MODE == OUT_SWIGLU ? (N / 2) / 128 : (N + kBN - 1) / kBN;
  if (n_tiles > kMaxNTiles) return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d too large", what, N);
  // Upper bound on the m-tiles: sum_g ceil(M_g / BM) <= floor(M / BM) + G, and
  // every m-tile holds at least one row.
  int64_t mt_bound = M / kBM + G;
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
  grouped_gemm_kernel<MODE><<<(unsigned)(8 * wg_per_xcd), kThreads, 0, st>>>(
      aq, as, a_row, (int)a_rows, bq, bs, offsets, G, N, K, n_tiles, (int)wg_per_xcd, out, hs);
  return after_launch(what, st);
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

extern "C" moe_status grouped_gemm_fp8_blockscaled(const uint8_t* aq, const float* as,
                                                   const int32_t* a_row, int64_t a_rows,
                                                   const uint8_t* bq, const float* bs,
                                                   const int32_t* group_offsets, int32_t G,
                                                   int64_t M, int32_t N, int32_t K, void* c,
                                                   moe_dtype c_dtype, void* stream) {
  clear_detail();
  MOE_REQUIRE(c_dtype == MOE_F32 || c_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "c_dtype %d", (int)c_dtype);
  moe_status stt = check_gemm_args(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(c, MOE_ERR_NULL, "c is required");
  MOE_REQUIRE(aligned(c, 16), MOE_ERR_ALIGN, "c needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  if (c_dtype == MOE_F32)
    return launch_gemm<OUT_F32>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K, c, nullptr, st,
                                "grouped_gemm_fp8_blockscaled");
  return launch_gemm<OUT_BF16>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, N, K, c, nullptr, st,
                               "grouped_gemm_fp8_blockscaled");
}

extern "C" moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, const int32_t* a_row,
                                              int64_t a_rows, const uint8_t* bq, const float* bs,
                                              const int32_t* group_offsets, int32_t G, int64_t M,
                                              int32_t I, int32_t K, uint8_t* hq, float* hs,
                                              void* stream) {
  clear_detail();
  MOE_REQUIRE(I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "I=%d must be a positive multiple of 128", I);
  moe_status stt = check_gemm_args(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, 2 * I, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(hq && hs, MOE_ERR_NULL, "hq and hs are required");
  MOE_REQUIRE(aligned(hq, 16) && aligned(hs, 4), MOE_ERR_ALIGN, "hq needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  return launch_gemm<OUT_SWIGLU>(aq, as, a_row, a_rows, bq, bs, group_offsets, G, M, 2 * I, K, hq, hs, st,
                                 "grouped_gemm_fp8_swiglu");
}
