// Per-expert permutation of (token, slot) pairs: a stable counting sort with
// no token dropped and no padding ([DSV3-MOE] no token dropping; the grouped
// expert GEMM consumes the rows of each expert contiguously).
//
// Deterministic by construction (no order-dependent atomics):
//   1. count   : per block of 256 tokens, an LDS histogram of expert ids
//                (integer atomics: the counts do not depend on order);
//   2. scan    : one workgroup turns the [blocks, E] counts into expert
//                offsets and per-(block, expert) base rows (each expert's
//                blocks split over 1024 / E' threads, E' = E rounded up to a
//                power of two);
//   3. rank    : per token block, an LDS bit matrix [E][256] marks which
//                tokens picked each expert; the rank of token t inside
//                expert e is the popcount of e's bits below t, so rows follow
//                ascending token id;
//   4. gather  : one wavefront per destination row copies the row's FP8 codes
//                (16-byte vectors) and its 1x128 scales.
#include "device_common.h"
#include "host_common.h"

#include <mutex>

namespace moefp8 {
namespace {

constexpr int kBT = 256;  // tokens per block

__global__ __launch_bounds__(kBT) void permute_count_kernel(const int* __restrict__ idx, int T,
                                                            int K, int E,
                                                            int* __restrict__ counts) {
  extern __shared__ int hist[];  // [E]
  for (int e = threadIdx.x; e < E; e += kBT) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kBT + threadIdx.x;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicAdd(&hist[idx[(int64_t)t * K + k]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBT) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 1024 threads.  Experts are padded to Ep (a power of two)
// and each gets P = 1024 / Ep threads, thread (e, part) summing a run of
// consecutive blocks, so the count rows stream in with P-fold parallelism.
__global__ __launch_bounds__(1024) void permute_scan_kernel(const int* __restrict__ counts,
                                                            int nblk, int E, int Ep,
                                                            int* __restrict__ base,
                                                            int* __restrict__ offsets) {
  __shared__ int sSeg[1024];  // [part][Ep]: a run's sum, then its exclusive prefix
  __shared__ int sScan[1024];
  const int tid = threadIdx.x;
  const int P = 1024 / Ep, e = tid % Ep, part = tid / Ep;
  const int S = (nblk + P - 1) / P;
  const int b0 = min(part * S, nblk), b1 = min(b0 + S, nblk);
  int seg = 0;
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = counts[(int64_t)(b + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) seg += v[j];
    }
    for (; b < b1; ++b) seg += counts[(int64_t)b * E + e];
  }
  sSeg[tid] = seg;
  __syncthreads();
  // per expert: exclusive prefix over its runs, and its total
  int tot = 0;
  if (tid < Ep) {
    for (int p = 0; p < P; ++p) {
      const int v = sSeg[p * Ep + tid];
      sSeg[p * Ep + tid] = tot;
      tot += v;
    }
  }
  // inclusive Hillis-Steele scan of the totals over the Ep experts
  sScan[tid] = tid < Ep ? tot : 0;
  __syncthreads();
  for (int d = 1; d < Ep; d <<= 1) {
    const int v = (tid < Ep && tid >= d) ? sScan[tid - d] : 0;
    __syncthreads();
    if (tid < Ep) sScan[tid] += v;
    __syncthreads();
  }
  const int total = sScan[Ep - 1];
  __syncthreads();                  // every thread has read the total
  if (tid < Ep) sScan[tid] -= tot;  // exclusive: expert tid's first row
  __syncthreads();
  if (tid < E) offsets[tid] = sScan[tid];
  if (tid == 0) offsets[E] = total;
  if (e < E) {
    int run = sScan[e] + sSeg[part * Ep + e];
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = counts[(int64_t)(b + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        base[(int64_t)(b + j) * E + e] = run;
        run += v[j];
      }
    }
    for (; b < b1; ++b) {
      base[(int64_t)b * E + e] = run;
      run += counts[(int64_t)b * E + e];
    }
  }
}

__global__ __launch_bounds__(kBT) void permute_rank_kernel(const int* __restrict__ idx, int T,
                                                           int K, int E,
                                                           const int* __restrict__ base,
                                                           int* __restrict__ dst_row,
                                                           int* __restrict__ src_token) {
  extern __shared__ uint32_t bits[];  // [E][kBT / 32]
  constexpr int W = kBT / 32;
  for (int i = threadIdx.x; i < E * W; i += kBT) bits[i] = 0;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kBT + tl;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicOr(&bits[idx[(int64_t)t * K + k] * W + tl / 32], 1u << (tl % 32));
  __syncthreads();
  if (t < T) {
    const int w = tl / 32;
    const uint32_t below = (1u << (tl % 32)) - 1u;
    for (int k = 0; k < K; ++k) {
      const int e = idx[(int64_t)t * K + k];
      const uint32_t* row = bits + e * W;
      int rank = __popc(row[w] & below);
      for (int j = 0; j < w; ++j) rank += __popc(row[j]);
      const int d = base[(int64_t)blockIdx.x * E + e] + rank;
      dst_row[(int64_t)t * K + k] = d;
      src_token[d] = t;
    }
  }
}

// 4 wavefronts per workgroup, one destination row each.
__global__ __launch_bounds__(256) void permute_gather_kernel(const int* __restrict__ src_token,
                                                             int64_t rows, int H,
                                                             const uint8_t* __restrict__ xq,
                                                             const float* __restrict__ xs,
                                                             uint8_t* __restrict__ aq,
                                                             float* __restrict__ as) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int64_t t = src_token[r];
  const uint4* s = reinterpret_cast<const uint4*>(xq + t * H);
  uint4* d = reinterpret_cast<uint4*>(aq + r * H);
  const int nv = H / 16;
  for (int i = lane; i < nv; i += 64) d[i] = s[i];
  const int ns = H / 128;
  for (int i = lane; i < ns; i += 64) as[r * ns + i] = xs[t * ns + i];
}

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_permute_workspace_size(int32_t T, int32_t K, int32_t E, size_t* bytes) {
  clear_detail();
  MOE_REQUIRE(bytes, MOE_ERR_NULL, "bytes is required");
  MOE_REQUIRE(T >= 0 && K >= 1 && E >= 1 && K <= E, MOE_ERR_SHAPE, "T=%d K=%d E=%d", T, K, E);
  MOE_REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "E=%d > 1024", E);
  const size_t nblk = ((size_t)T + kBT - 1) / kBT;
  *bytes = 2 * nblk * (size_t)E * sizeof(int32_t) + 256;
  return MOE_OK;
}

namespace moefp8 {
namespace {

// Argument checks shared by both entry points (host only).
moe_status check_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E, const uint8_t* xq,
                         const float* xs, int32_t H, int32_t* expert_offsets, int32_t* dst_row,
                         int32_t* src_token, uint8_t* aq, float* as, bool* gather) {
  MOE_REQUIRE(T >= 0 && K >= 1 && E >= 1 && K <= E, MOE_ERR_SHAPE, "T=%d K=%d E=%d (need 1<=K<=E)", T, K, E);
  MOE_REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "E=%d > 1024", E);
  MOE_REQUIRE((int64_t)T * K < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*K too large");
  *gather = xq != nullptr || xs != nullptr || aq != nullptr || as != nullptr;
  if (*gather) {
    MOE_REQUIRE(xq && xs && aq && as, MOE_ERR_NULL, "xq, xs, aq and as must be all set or all NULL");
    MOE_REQUIRE(H > 0 && H % 128 == 0, MOE_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
    MOE_REQUIRE(aligned(xq, 16) && aligned(aq, 16) && aligned(xs, 4) && aligned(as, 4), MOE_ERR_ALIGN,
                "xq and aq need 16-byte alignment");
  }
  MOE_REQUIRE(expert_offsets, MOE_ERR_NULL, "expert_offsets is required");
  MOE_REQUIRE(T == 0 || (topk_idx && dst_row && src_token), MOE_ERR_NULL,
              "topk_idx, dst_row and src_token are required");
  MOE_REQUIRE(aligned(topk_idx, 4) && aligned(expert_offsets, 4) && aligned(dst_row, 4) && aligned(src_token, 4),
              MOE_ERR_ALIGN, "index arrays need 4-byte alignment");
  return MOE_OK;
}

// The four launches; `workspace` holds counts [nblk, E] then base [nblk, E]
// (every element written by the count and scan kernels before it is read,
// so nothing needs clearing).
moe_status launch_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E, const uint8_t* xq,
                          const float* xs, int32_t H, int32_t* expert_offsets, int32_t* dst_row,
                          int32_t* src_token, uint8_t* aq, float* as, bool gather, void* workspace,
                          hipStream_t st, const char* what) {
  const int nblk = (int)(((int64_t)T + kBT - 1) / kBT);
  int* counts = reinterpret_cast<int*>(workspace);
  int* base = counts + (size_t)nblk * E;
  if (nblk > 0)
    permute_count_kernel<<<nblk, kBT, E * sizeof(int), st>>>(topk_idx, T, K, E, counts);
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  permute_scan_kernel<<<1, 1024, 0, st>>>(counts, nblk, E, Ep, base, expert_offsets);
  if (nblk > 0)
    permute_rank_kernel<<<nblk, kBT, E * (kBT / 32) * sizeof(uint32_t), st>>>(topk_idx, T, K, E, base,
                                                                              dst_row, src_token);
  const int64_t rows = (int64_t)T * K;
  if (gather && rows > 0)
    permute_gather_kernel<<<ceil_div_u(rows, 4), 256, 0, st>>>(src_token, rows, H, xq, xs, aq, as);
  return after_launch(what, st);
}

// Scratch of moe_permute_noalloc: a file-scope device array (one copy per
// GPU, held until the process ends).  Host code never uses the array's name
// as an address: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept here.
constexpr size_t kPermuteScratchBytes = size_t(4) << 20;
__device__ __align__(256) uint8_t scratch[kPermuteScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status permute_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moefp8

extern "C" moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E,
                                  const uint8_t* xq, const float* xs, int32_t H,
                                  int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                                  uint8_t* aq, float* as, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  clear_detail();
  bool gather = false;
  moe_status stt = check_permute(topk_idx, T, K, E, xq, xs, H, expert_offsets, dst_row, src_token, aq, as,
                                 &gather);
  if (stt != MOE_OK) return stt;
  size_t need = 0;
  moe_permute_workspace_size(T, K, E, &need);
  MOE_REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  MOE_REQUIRE(workspace, MOE_ERR_NULL, "workspace is required");
  MOE_REQUIRE(aligned(workspace, 16), MOE_ERR_ALIGN, "workspace needs 16-byte alignment");
  return launch_permute(topk_idx, T, K, E, xq, xs, H, expert_offsets, dst_row, src_token, aq, as, gather,
                        workspace, as_stream(stream), "moe_permute");
}

extern "C" moe_status moe_permute_noalloc(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E,
                                          const uint8_t* xq, const float* xs, int32_t H,
                                          int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                                          uint8_t* aq, float* as, void* stream) {
  clear_detail();
  bool gather = false;
  moe_status stt = check_permute(topk_idx, T, K, E, xq, xs, H, expert_offsets, dst_row, src_token, aq, as,
                                 &gather);
  if (stt != MOE_OK) return stt;
  size_t need = 0;
  moe_permute_workspace_size(T, K, E, &need);
  MOE_REQUIRE(need <= kPermuteScratchBytes, MOE_ERR_WORKSPACE,
              "T=%d E=%d needs %zu bytes of scratch; the static scratch holds %zu (use moe_permute)", T, E,
              need, kPermuteScratchBytes);
  void* ws = nullptr;
  stt = permute_scratch(&ws);
  if (stt != MOE_OK) return stt;
  return launch_permute(topk_idx, T, K, E, xq, xs, H, expert_offsets, dst_row, src_token, aq, as, gather, ws,
                        as_stream(stream), "moe_permute_noalloc");
}
