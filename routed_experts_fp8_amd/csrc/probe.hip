// Measurement helper, not a step of the layer: the matrix cores' own FP8
// ceiling on this device, so that the grouped GEMMs' rates can be read
// against a measured figure beside the datasheet's.
//
// moe_probe_mfma_fp8_kernel: every wave keeps kChains independent
// accumulator chains of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (each instruction
// 16 x 16 x 128 multiply-adds = 65536 flops) on operands held in registers,
// iters instructions per chain with no memory traffic inside the loop, then
// writes one sum per lane so the work cannot be removed.  With every code of
// both operands equal to `code` (E4M3 value v), each instruction adds 128 v^2
// to every accumulator element, so a lane's sum is exactly
// kChains * 4 * 128 * v^2 * iters while that stays an integer below 2^24.
#include "host_common.h"
#include "lds_dma.h"

namespace moefp8 {
namespace {

constexpr int kChains = 8;

__global__ void moe_probe_mfma_fp8_kernel(uint32_t code, int64_t iters, float* __restrict__ out) {
  const uint32_t word = code * 0x01010101u;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (int)word, b[i] = (int)word;
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_probe_mfma_fp8(uint8_t code, int64_t iters, int32_t blocks, int32_t waves_per_block,
                                         float* out, double* flops, void* stream) {
  clear_detail();
  MOE_REQUIRE(out && flops, MOE_ERR_NULL, "out and flops are required");
  MOE_REQUIRE(iters >= 0 && iters <= (int64_t(1) << 32), MOE_ERR_SHAPE, "iters=%lld (0..2^32)", (long long)iters);
  MOE_REQUIRE(blocks >= 1 && blocks <= (1 << 20), MOE_ERR_SHAPE, "blocks=%d (1..2^20)", blocks);
  MOE_REQUIRE(waves_per_block >= 1 && waves_per_block <= 16, MOE_ERR_SHAPE, "waves_per_block=%d (1..16)",
              waves_per_block);
  MOE_REQUIRE(aligned(out, 4), MOE_ERR_ALIGN, "out needs 4-byte alignment");
  *flops = (double)blocks * waves_per_block * (double)iters * kChains * 65536.0;
  hipStream_t s = as_stream(stream);
  moe_probe_mfma_fp8_kernel<<<blocks, 64 * waves_per_block, 0, s>>>(code, iters, out);
  return after_launch("moe_probe_mfma_fp8", s);
}
