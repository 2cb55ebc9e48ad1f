// Bit-exact transpose of block-quantised weights, codes and scale grid
// ([KANANA-FP8]: keep only the forward FP8 weights; the backward pass
// transposes the block-quantised weights instead of re-quantising).
//
// One 256-thread workgroup moves one 128x128-byte block: 16-byte coalesced
// loads (8 lanes per 128-byte row segment) into LDS, then the transposed
// write of device_common.h (16-row x 4-column byte patches per thread,
// 16-byte stores).
#include "device_common.h"
#include "host_common.h"

namespace moefp8 {
namespace {

__global__ __launch_bounds__(256) void block_transpose_kernel(const uint8_t* __restrict__ q,
                                                              const float* __restrict__ s,
                                                              int rows, int cols,
                                                              uint8_t* __restrict__ qt,
                                                              float* __restrict__ st) {
  __shared__ uint32_t tile[128 * kTilePitch / 4];
  const int bc = cols / 128, br = rows / 128;
  const int64_t blk = blockIdx.x;
  const int bj = (int)(blk % bc);
  const int bi = (int)((blk / bc) % br);
  const int64_t g = blk / ((int64_t)bc * br);
  const int64_t plane = (int64_t)rows * cols;
  const uint8_t* src = q + g * plane + (int64_t)bi * 128 * cols + bj * 128;
  uint8_t* dst = qt + g * plane + (int64_t)bj * 128 * rows + bi * 128;
  const int tid = threadIdx.x;

  uint4 in[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + tid;
    const int r = id >> 3, c16 = id & 7;
    in[i] = load16_nt(src + (int64_t)r * cols + c16 * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + tid;
    const int r = id >> 3, c16 = id & 7;
    uint32_t* p = tile + (r * kTilePitch + c16 * 16) / 4;
    p[0] = in[i].x;
    p[1] = in[i].y;
    p[2] = in[i].z;
    p[3] = in[i].w;
  }
  __syncthreads();

  write_block_transposed(tile, dst, rows, tid);
  if (tid == 0) {
    // scale grid: s[g][bi][bj] -> st[g][bj][bi]
    st[g * (int64_t)br * bc + (int64_t)bj * br + bi] = s[blk];
  }
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status fp8_block_transpose(const uint8_t* q, const float* scale, int32_t G,
                                          int32_t rows, int32_t cols, uint8_t* qt, float* scale_t,
                                          void* stream) {
  clear_detail();
  MOE_REQUIRE(G >= 0 && rows > 0 && cols > 0 && rows % 128 == 0 && cols % 128 == 0, MOE_ERR_SHAPE,
              "G=%d rows=%d cols=%d (rows, cols positive multiples of 128)", G, rows, cols);
  MOE_REQUIRE(elems_ok((int64_t)G * rows, cols), MOE_ERR_UNSUPPORTED, "G=%d x %d x %d above 2^40 elements", G,
              rows, cols);
  if (G == 0) return MOE_OK;
  MOE_REQUIRE(q && scale && qt && scale_t, MOE_ERR_NULL, "q, scale, qt and scale_t are required");
  MOE_REQUIRE(aligned(q, 16) && aligned(qt, 16) && aligned(scale, 4) && aligned(scale_t, 4),
              MOE_ERR_ALIGN, "q and qt need 16-byte alignment, scales 4-byte");
  const int64_t nblk = (int64_t)G * (rows / 128) * (cols / 128);
  MOE_REQUIRE(nblk < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many blocks (%lld)", (long long)nblk);
  hipStream_t st = as_stream(stream);
  block_transpose_kernel<<<(unsigned)nblk, 256, 0, st>>>(q, scale, rows, cols, qt, scale_t);
  return after_launch("fp8_block_transpose", st);
}
