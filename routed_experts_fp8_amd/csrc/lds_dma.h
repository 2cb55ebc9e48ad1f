// Direct global -> LDS operand staging for the gfx950 FP8 matrix kernels
// (the grouped GEMM and the weight-gradient GEMM): the load instructions
// and the operand read of one V_MFMA_SCALE_F32_16X16X128_F8F6F4 fragment
// from 128-byte LDS rows whose 16-byte pieces are XOR-swizzled (logical
// piece c16 of row r sits at byte 128 r + 16 (c16 ^ (r & 7)); the loads
// apply it on the global side, since the DMA fixes lane -> LDS address).
#pragma once

#include "device_common.h"

namespace moefp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Direct global -> LDS loads (gfx950 global_load_lds_dword[x4]): lane i's
// 16 (4) bytes, read from sbase + voff_i (scalar base, per-lane 32-bit
// offset), land at LDS address `lds` + 16 i (4 i).  Issued from inline
// assembly so that the compiler's wait-count pass does not track them: its
// alias tracking of LDS DMA is coarse and would otherwise force every LDS
// read in a K loop to wait for ALL outstanding DMA, serialising the ring.
// The kernels wait for these loads themselves (s_waitcnt vmcnt + s_barrier)
// and keep no compiler-visible vector loads in flight while they do; stores
// issued after the loads can only delay such a wait, never satisfy it early
// (loads complete in issue order, and every store adds to the count).  The
// instructions have no destination registers; the address VGPRs are read
// at issue.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" : : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// s_waitcnt immediate that waits until at most n (< 16) vector-memory
// operations of this wave are outstanding (LDS and export counts untouched).
constexpr int vmcnt_imm(int n) { return 0x0F70 | n; }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// accesses, not for its vector-memory loads (DMA stays in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A fragment's lane reads row 16 r0 + lane % 16, bytes [32q, 32q + 32) of
// the 128-byte chunk (q = lane / 16).  Its row & 7 == lane & 7, so the
// swizzled byte offsets of its two 16-byte pieces (logical pieces 2q and
// 2q + 1) are the same for every row block:
// lane_lo = 128 (lane % 16) + 16 (2q ^ (lane & 7)), lane_hi = lane_lo ^ 16.
// The row block then enters as an immediate offset.
__device__ __forceinline__ uint32_t frag_lane_lo(int lane) {
  return (uint32_t)((lane & 15) * 128 + (((2 * (lane >> 4)) ^ (lane & 7)) << 4));
}
__device__ __forceinline__ v8i lds_operand(const uint8_t* rows16, uint32_t lane_lo, uint32_t lane_hi) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(rows16 + lane_lo);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(rows16 + lane_hi);
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// One 128-wide chunk of FP8 E4M3 x E4M3 dot products on the matrix core
// (format selectors 0, 0; no block-exponent scaling), zero accumulator in.
__device__ __forceinline__ v4f mfma_chunk(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

}  // namespace moefp8
