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
//    float32 result is exactly the chunk partial P_kb.  The promotion is one
//    VALU fused multiply-add per output per chunk:
//    acc = fma(P_kb, sa * sb, acc), in chunk order.
//  * The token dimension sits on the instruction's column axis and weight
//    rows on its row axis: every lane's 4 outputs share one token (one sa per
//    lane per chunk) and 4 consecutive weight rows inside one 128-row block
//    (one sb per wave per chunk, a scalar load).
//  * A workgroup owns a BM x BN tile of one group; 4 wavefronts each own a
//    64 x 64 sub-tile (4 x 4 instruction tiles).  K advances one 128-byte
//    chunk at a time through a double-buffered LDS stage filled with
//    16-byte loads (8 lanes per 128-byte row segment, coalesced); rows are
//    stored with a 16-byte XOR swizzle so the operand reads (32 bytes per
//    lane) spread over the LDS banks.
//  * Ragged groups: token rows past the group's end are clamped on load and
//    never stored; 16-row instruction tiles that lie entirely past the end
//    are skipped, so a group with M_g rows costs ceil(M_g / 16) tiles of
//    matrix work, not BM.
//  * Tile table on the device, no host sync: every workgroup reads the group
//    offsets, counts each group's m-tiles, prefix-sums them in LDS and finds
//    its own tile, so the grid is sized from the host-known bound
//    floor(M / BM) + G m-tiles.
//  * XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
//    block b is remapped to logical tile xcd * ceil(tiles / 8) + b / 8.  Each
//    XCD then sweeps a contiguous run of (group, n-tile, m-tile) tiles:
//    m-tiles sharing one weight slab and n-tiles sharing one activation tile
//    run together on one XCD and share its L2.
//  * Fused SwiGLU (grouped_gemm_fp8_swiglu): the B tile is the gate block c
//    (weight rows 128c..) stacked on the up block c (rows I + 128c..), and
//    every wave holds matching gate and up rows, so h = silu(g) * u is formed
//    in registers; the 1x128 amax of h along I is reduced across lanes and
//    waves through LDS, and only the FP8 codes and scales of h are written.
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_SWIGLU = 2 };

constexpr int kThreads = 256;
constexpr int kMaxGroups = 1024;

__device__ __forceinline__ v4f mfma_chunk(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // FP8 E4M3 x FP8 E4M3 (format selectors 0, 0), no block-exponent scaling.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Byte offset of 16-byte piece c16 of row r inside a [rows][128] LDS stage.
__device__ __forceinline__ int swz(int r, int c16) { return r * 128 + ((c16 ^ (r & 7)) << 4); }

// 32 bytes of row r starting at byte 32 * q (q = lane / 16) -> v8i.
__device__ __forceinline__ v8i lds_operand(const uint8_t* stage, int r, int q) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(stage + swz(r, 2 * q));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(stage + swz(r, 2 * q + 1));
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ aq, const float* __restrict__ as, const uint8_t* __restrict__ bq,
    const float* __restrict__ bs, const int* __restrict__ offsets, int G, int N, int K, int n_tiles,
    void* __restrict__ out, float* __restrict__ hs_out) {
  static_assert(WM * WN == 4, "4 wavefronts");
  constexpr int WTM = BM / WM;     // tokens per wave
  constexpr int WTN = BN / WN;     // weight rows per wave
  constexpr int NTM = WTM / 16;    // instruction tiles along tokens
  constexpr int NTN = WTN / 16;    // instruction tiles along weight rows
  constexpr bool kFused = MODE == OUT_SWIGLU;
  static_assert(!kFused || BN == 256, "fused tile = 128 gate rows + 128 up rows");
  static_assert(kFused || WTN <= 128, "a wave's rows must sit in one 128-row block");
  constexpr int APT = BM * 8 / kThreads;  // 16-byte A pieces per thread per chunk
  constexpr int BPT = BN * 8 / kThreads;  // 16-byte B pieces per thread per chunk
  static_assert(APT >= 1 && BPT >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * 128];
  __shared__ float sSA[2][BM];
  __shared__ int sP[kMaxGroups + 1];
  __shared__ int sOff[kMaxGroups + 1];
  __shared__ int sScan[kThreads];
  __shared__ float sAmax[kFused ? WN : 1][kFused ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- tile table: m-tiles per group, prefix sums, this block's tile ----
  {
    int local = 0;
    int mt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = tid * 4 + i;
      mt[i] = 0;
      if (g < G) {
        const int o0 = offsets[g], o1 = offsets[g + 1];
        sOff[g] = o0;
        mt[i] = (o1 - o0 + BM - 1) / BM;
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
    for (int i = 0; i < 4; ++i) {
      const int g = tid * 4 + i;
      if (g < G) sP[g] = run;
      run += mt[i];
    }
    if (tid == kThreads - 1) sP[G] = sScan[kThreads - 1];
    __syncthreads();
  }
  const int total_mt = sP[G];
  const int total = total_mt * n_tiles;
  const int chunk = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= chunk) return;
  const int lid = (blockIdx.x & 7) * chunk + slot;
  if (lid >= total) return;
  int g;
  {
    int lo = 0, hi = G;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sP[mid] * n_tiles <= lid) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
  const int mt_g = sP[g + 1] - sP[g];
  const int local_id = lid - sP[g] * n_tiles;
  const int n_tile = local_id / mt_g;
  const int m_tile = local_id % mt_g;
  const int row0 = sOff[g] + m_tile * BM;
  const int rows_valid = min(BM, sOff[g + 1] - row0);
  const int KB = K / 128;
  const int I = N / 2;  // fused mode: gate rows [0, I), up rows [I, 2I)

  const int wn = wave % WN, wm = wave / WN;
  // 128-row weight blocks of this wave's rows (gate / up blocks in fused mode)
  const int blk0 = kFused ? n_tile : (n_tile * BN + wn * WTN) / 128;
  const int blk1 = kFused ? I / 128 + n_tile : blk0;

  const uint8_t* bq_g = bq + (int64_t)g * N * K;
  const float* bs_g = bs + (int64_t)g * (N / 128) * KB;

  // ---- global -> register staging of one chunk (fully unrolled) ----
  u32x4 ra[APT], rb[BPT];
  float rsa = 0.f;
  float rsb0 = 0.f, rsb1 = 0.f;  // weight-block scales of the staged chunk (wave-uniform)
  const uint8_t* a_src[APT];      // per-piece row base pointers (chunk 0)
  const uint8_t* b_src[BPT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int p = i * kThreads + tid;
    const int64_t grow = row0 + min(p >> 3, rows_valid - 1);
    a_src[i] = aq + grow * K + (p & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int p = i * kThreads + tid;
    const int r = p >> 3;
    const int wrow = kFused ? (r < 128 ? n_tile * 128 + r : I + n_tile * 128 + (r - 128))
                            : n_tile * BN + r;
    b_src[i] = bq_g + (int64_t)wrow * K + (p & 7) * 16;
  }
  const float* sa_src = as + (int64_t)(row0 + min(tid, rows_valid - 1)) * KB;
  const float* sb_src0 = bs_g + (int64_t)blk0 * KB;
  const float* sb_src1 = bs_g + (int64_t)blk1 * KB;

#define MOE_LOAD_CHUNK(kb)                                                        \
  do {                                                                            \
    _Pragma("unroll") for (int i = 0; i < APT; ++i) ra[i] =                       \
        *reinterpret_cast<const u32x4*>(a_src[i] + (kb) * 128);                   \
    _Pragma("unroll") for (int i = 0; i < BPT; ++i) rb[i] =                       \
        *reinterpret_cast<const u32x4*>(b_src[i] + (kb) * 128);                   \
    if (tid < BM) rsa = sa_src[kb];                                               \
    rsb0 = sb_src0[kb];                                                           \
    rsb1 = sb_src1[kb];                                                           \
  } while (0)
#define MOE_STORE_CHUNK(s)                                                        \
  do {                                                                            \
    _Pragma("unroll") for (int i = 0; i < APT; ++i) {                             \
      const int p = i * kThreads + tid;                                           \
      *reinterpret_cast<u32x4*>(&sA[s][swz(p >> 3, p & 7)]) = ra[i];              \
    }                                                                             \
    _Pragma("unroll") for (int i = 0; i < BPT; ++i) {                             \
      const int p = i * kThreads + tid;                                           \
      *reinterpret_cast<u32x4*>(&sB[s][swz(p >> 3, p & 7)]) = rb[i];              \
    }                                                                             \
    if (tid < BM) sSA[s][tid] = rsa;                                              \
  } while (0)

  // ---- wave geometry ----
  const int q = lane >> 4, l16 = lane & 15;
  int brow[NTN];  // B-tile row of n-tile i for this lane
#pragma unroll
  for (int i = 0; i < NTN; ++i) {
    if (kFused) {
      constexpr int half = NTN / 2;
      brow[i] = (i < half ? 0 : 128) + wn * (128 / WN) + 16 * (i % half) + l16;
    } else {
      brow[i] = wn * WTN + 16 * i + l16;
    }
  }
  int n_active = 0;  // instruction tiles along tokens holding a valid row
#pragma unroll
  for (int j = 0; j < NTM; ++j)
    if (wm * WTM + 16 * j < rows_valid) n_active = j + 1;

  v4f acc[NTN][NTM];
#pragma unroll
  for (int i = 0; i < NTN; ++i)
#pragma unroll
    for (int j = 0; j < NTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  MOE_LOAD_CHUNK(0);
  float sb0 = rsb0, sb1 = rsb1;
  MOE_STORE_CHUNK(0);
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const int s = kb & 1;
    if (kb + 1 < KB) MOE_LOAD_CHUNK(kb + 1);
    v8i a_op[NTN];
#pragma unroll
    for (int i = 0; i < NTN; ++i) a_op[i] = lds_operand(sB[s], brow[i], q);
#pragma unroll
    for (int j = 0; j < NTM; ++j) {
      if (j < n_active) {
        const int arow = wm * WTM + 16 * j + l16;
        const v8i b_op = lds_operand(sA[s], arow, q);
        const float sa = sSA[s][arow];
        const float sc0 = sa * sb0;
        const float sc1 = kFused ? sa * sb1 : sc0;
#pragma unroll
        for (int i = 0; i < NTN; ++i) {
          const v4f p = mfma_chunk(a_op[i], b_op);
          const float sc = (kFused && i >= NTN / 2) ? sc1 : sc0;
          acc[i][j][0] = __builtin_fmaf(p[0], sc, acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(p[1], sc, acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(p[2], sc, acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(p[3], sc, acc[i][j][3]);
        }
      }
    }
    if (kb + 1 < KB) {
      MOE_STORE_CHUNK(s ^ 1);
      sb0 = rsb0;
      sb1 = rsb1;
    }
    __syncthreads();
  }

#undef MOE_LOAD_CHUNK
#undef MOE_STORE_CHUNK

  // ---- epilogue ----
  if constexpr (!kFused) {
#pragma unroll
    for (int j = 0; j < NTM; ++j) {
      const int mloc = wm * WTM + 16 * j + l16;
      if (j < n_active && mloc < rows_valid) {
        const int64_t m = row0 + mloc;
#pragma unroll
        for (int i = 0; i < NTN; ++i) {
          const int n = n_tile * BN + wn * WTN + 16 * i + 4 * q;
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
    constexpr int HALF = NTN / 2;
    // h = silu(g) * u into the gate accumulators; per-token amax
#pragma unroll
    for (int j = 0; j < NTM; ++j) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < HALF; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h = spec_silu(acc[i][j][v]) * acc[i + HALF][j][v];
          acc[i][j][v] = h;
          amax = fmaxf(amax, fabsf(h));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      if (q == 0) sAmax[wn][wm * WTM + 16 * j + l16] = amax;
    }
    __syncthreads();
    const int Ih = I;  // h row length
#pragma unroll
    for (int j = 0; j < NTM; ++j) {
      const int mloc = wm * WTM + 16 * j + l16;
      if (j < n_active && mloc < rows_valid) {
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < WN; ++w) amax = fmaxf(amax, sAmax[w][mloc]);
        const float sc = scale_from_amax(amax);
        const int64_t m = row0 + mloc;
        uint8_t* hq = reinterpret_cast<uint8_t*>(out);
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
          const int col = n_tile * 128 + wn * (128 / WN) + 16 * i + 4 * q;
          const uint32_t w = quantize(acc[i][j][0], sc) | (quantize(acc[i][j][1], sc) << 8) |
                             (quantize(acc[i][j][2], sc) << 16) | (quantize(acc[i][j][3], sc) << 24);
          *reinterpret_cast<uint32_t*>(hq + m * Ih + col) = w;
        }
        if (wn == 0 && q == 0) hs_out[m * (Ih / 128) + n_tile] = sc;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int MODE>
moe_status launch_gemm(const uint8_t* aq, const float* as, const uint8_t* bq, const float* bs,
                       const int* offsets, int G, int64_t M, int N, int K, void* out, float* hs,
                       hipStream_t st, const char* what) {
  const int n_tiles = MODE == OUT_SWIGLU ? (N / 2) / 128 : N / BN;
  int64_t mt_bound = M / BM + G;
  if (mt_bound > M) mt_bound = M;
  const int64_t tiles = mt_bound * n_tiles;
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", what);
  if (grid == 0) return MOE_OK;
  grouped_gemm_kernel<BM, BN, WM, WN, MODE>
      <<<(unsigned)grid, kThreads, 0, st>>>(aq, as, bq, bs, offsets, G, N, K, n_tiles, out, hs);
  return after_launch(what, st);
}

moe_status check_gemm_args(const uint8_t* aq, const float* as, const uint8_t* bq, const float* bs,
                           const int32_t* offsets, int32_t G, int64_t M, int32_t N, int32_t K) {
  MOE_REQUIRE(G >= 1 && M >= 0 && N > 0 && K > 0, MOE_ERR_SHAPE, "G=%d M=%lld N=%d K=%d", G,
              (long long)M, N, K);
  MOE_REQUIRE(G <= kMaxGroups, MOE_ERR_UNSUPPORTED, "G=%d > %d", G, kMaxGroups);
  MOE_REQUIRE(N % 128 == 0 && K % 128 == 0, MOE_ERR_SHAPE, "N=%d and K=%d must be multiples of 128", N, K);
  MOE_REQUIRE(M < (1LL << 31), MOE_ERR_UNSUPPORTED, "M too large");
  MOE_REQUIRE(offsets, MOE_ERR_NULL, "group_offsets is required");
  MOE_REQUIRE(aligned(offsets, 4), MOE_ERR_ALIGN, "group_offsets needs 4-byte alignment");
  if (M == 0) return MOE_OK;
  MOE_REQUIRE(aq && as && bq && bs, MOE_ERR_NULL, "aq, as, bq and bs are required");
  MOE_REQUIRE(aligned(aq, 16) && aligned(bq, 16) && aligned(as, 4) && aligned(bs, 4), MOE_ERR_ALIGN,
              "aq and bq need 16-byte alignment, scales 4-byte");
  return MOE_OK;
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status grouped_gemm_fp8_blockscaled(const uint8_t* aq, const float* as,
                                                   const uint8_t* bq, const float* bs,
                                                   const int32_t* group_offsets, int32_t G,
                                                   int64_t M, int32_t N, int32_t K, void* c,
                                                   moe_dtype c_dtype, void* stream) {
  clear_detail();
  MOE_REQUIRE(c_dtype == MOE_F32 || c_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "c_dtype %d", (int)c_dtype);
  moe_status stt = check_gemm_args(aq, as, bq, bs, group_offsets, G, M, N, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(c, MOE_ERR_NULL, "c is required");
  MOE_REQUIRE(aligned(c, 16), MOE_ERR_ALIGN, "c needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  if (c_dtype == MOE_F32)
    return launch_gemm<128, 128, 2, 2, OUT_F32>(aq, as, bq, bs, group_offsets, G, M, N, K, c, nullptr,
                                                st, "grouped_gemm_fp8_blockscaled");
  return launch_gemm<128, 128, 2, 2, OUT_BF16>(aq, as, bq, bs, group_offsets, G, M, N, K, c, nullptr,
                                               st, "grouped_gemm_fp8_blockscaled");
}

extern "C" moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, const uint8_t* bq,
                                              const float* bs, const int32_t* group_offsets,
                                              int32_t G, int64_t M, int32_t I, int32_t K,
                                              uint8_t* hq, float* hs, void* stream) {
  clear_detail();
  MOE_REQUIRE(I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "I=%d must be a positive multiple of 128", I);
  moe_status stt = check_gemm_args(aq, as, bq, bs, group_offsets, G, M, 2 * I, K);
  if (stt != MOE_OK || M == 0) return stt;
  MOE_REQUIRE(hq && hs, MOE_ERR_NULL, "hq and hs are required");
  MOE_REQUIRE(aligned(hq, 16) && aligned(hs, 4), MOE_ERR_ALIGN, "hq needs 16-byte alignment");
  hipStream_t st = as_stream(stream);
  return launch_gemm<64, 256, 1, 4, OUT_SWIGLU>(aq, as, bq, bs, group_offsets, G, M, 2 * I, K, hq, hs, st,
                                                "grouped_gemm_fp8_swiglu");
}
