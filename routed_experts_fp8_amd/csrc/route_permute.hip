// Routing and the per-expert permutation's index maps in one launch
// ([DSV3-MOE] section 2.1: top-K selection, no token dropped; [PANGU-MOGE]
// grouped selection; the operator-fusion item of the Pangu page's system
// optimisation section).  The results are those of moe_route followed by
// moe_permute, bit for bit.
//
// Workgroups (1024 threads; 512 when E > 512) take a ticket from a device
// counter as their first action; the ticket, not the workgroup index, picks
// the role:
//   tickets [0, nA)        routing block b: 64 tokens (16 wavefronts x 4
//                          tokens, or 8 x 8; route_device.h).  Each pick bumps an LDS
//                          histogram and sets the token's bit in an LDS bit
//                          row of its expert; after a barrier the block
//                          writes its counts row cnt[b][0..E) and, for every
//                          (token, slot), the rank of the token among the
//                          block's tokens that picked the same expert (a
//                          popcount of the bit row below the token) into
//                          dst_row.  The last routing block to finish (an
//                          arrival counter) scans: expert offsets from the
//                          per-expert totals, and base[b][e] = offsets[e] +
//                          the counts of expert e in blocks before b (each
//                          expert's blocks split over NT / E' threads, so
//                          the count rows stream in parallel); then it raises
//                          `ready`;
//   tickets [nA, nA + nC)  ranking: 512 tokens each; waits for `ready`, then
//                          dst_row[t, k] += base[t / 64][expert] and
//                          src_token[dst_row[t, k]] = t.
// Rows follow ascending token order inside each expert, as in moe_permute.
// A ranking workgroup only waits on routing workgroups, and every routing
// ticket was drawn before any ranking ticket, by a workgroup that was then
// already running: the wait always ends, whatever else occupies the GPU.
// It is still bounded (about a second); a wait that runs out writes nothing
// and counts itself in the header's `timeouts` word.
//
// Workspace: a 256-byte header {ticket, a_done, c_done, ready, timeouts},
// then cnt [nA][E] and base [nA][E] (written before they are read in every
// call).  The header must be zero before the first call; the last ranking
// workgroup to finish (with T == 0, the only workgroup) resets it, so every
// call leaves it zero again.
#include "device_common.h"
#include "host_common.h"
#include "route_device.h"

namespace moefp8 {
namespace {

// 1024 threads per workgroup; 512 when a lane holds 16 expert keys (E > 512),
// so the routing registers fit without spilling
template <int PL>
constexpr int rp_threads() { return PL > 8 ? 512 : 1024; }
constexpr int kRPMaxThreads = 1024;
constexpr int kRPBlock = 64;                       // tokens per routing block
constexpr int kRPRankTokens = 512;                 // tokens per ranking workgroup
constexpr int kRPHeaderBytes = 256;
constexpr int kRPSpinLimit = 1 << 23;  // x s_sleep(2) ~ 0.5-1 s

struct RPState {
  int ticket, a_done, c_done, ready, timeouts;
};

struct RPArgs {
  const float* logits;
  const float* bias;
  int T, E, K, G, Kp, mode, normalize;
  int* idx;
  float* gate;
  int* offsets;
  int* dst_row;
  int* src_token;
  RPState* state;
  int* cnt;   // [nA][E]
  int* base;  // [nA][E]
  int nA, nC, Ep;  // Ep: E rounded up to a power of two
};

__device__ __forceinline__ void rp_reset(RPState* s) {
  __hip_atomic_store(&s->ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&s->a_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&s->c_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&s->ready, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan of v over threads [0, n) (n a power of two, at
// most the block size; every thread of the block calls it); returns the
// exclusive prefix and the total in *total.
__device__ int rp_block_scan(int v, int n, int* sBuf, int* total) {
  const int tid = threadIdx.x;
  if (tid < n) sBuf[tid] = v;
  __syncthreads();
  for (int d = 1; d < n; d <<= 1) {
    const int a = (tid < n && tid >= d) ? sBuf[tid - d] : 0;
    __syncthreads();
    if (tid < n) sBuf[tid] += a;
    __syncthreads();
  }
  const int incl = tid < n ? sBuf[tid] : 0;
  *total = sBuf[n - 1];
  __syncthreads();
  return incl - v;
}

// Expert offsets and base rows (the last routing block; all NT threads).
// Experts are taken Ew = min(E', NT) at a time; each of a pass's experts has
// NT / Ew threads, each summing one run of blocks.
template <int NT>
__device__ void rp_scan(const RPArgs& a, int* sSeg, int* sBuf) {
  const int tid = threadIdx.x;
  const int Ew = min(a.Ep, NT), P = NT / Ew;
  const int e_in = tid % Ew, part = tid / Ew;
  const int S = (a.nA + P - 1) / P;
  const int b0 = min(part * S, a.nA), b1 = min(b0 + S, a.nA);
  const int* __restrict__ cnt = a.cnt;
  int* __restrict__ base = a.base;
  int carry = 0;
  for (int e0 = 0; e0 < a.Ep; e0 += Ew) {
    const int e = e0 + e_in;
    int seg = 0;
    if (e < a.E) {
      int b = b0;
      for (; b + 8 <= b1; b += 8) {
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = cnt[(int64_t)(b + j) * a.E + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) seg += v[j];
      }
      for (; b < b1; ++b) seg += cnt[(int64_t)b * a.E + e];
    }
    sSeg[tid] = seg;  // [part][Ew]
    __syncthreads();
    // per expert: exclusive prefix over the parts, and the expert's total
    int tot = 0;
    if (tid < Ew) {
      for (int p = 0; p < P; ++p) {
        const int v = sSeg[p * Ew + tid];
        sSeg[p * Ew + tid] = tot;
        tot += v;
      }
    }
    __syncthreads();
    int all = 0;
    const int off = carry + rp_block_scan(tot, Ew, sBuf, &all);  // expert offsets (threads < Ew)
    if (tid < Ew && e0 + tid < a.E) a.offsets[e0 + tid] = off;
    if (tid < Ew) sBuf[tid] = off;
    __syncthreads();
    if (e < a.E) {
      int run = sBuf[e_in] + sSeg[part * Ew + e_in];
      int b = b0;
      for (; b + 8 <= b1; b += 8) {
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = cnt[(int64_t)(b + j) * a.E + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          base[(int64_t)(b + j) * a.E + e] = run;
          run += v[j];
        }
      }
      for (; b < b1; ++b) {
        base[(int64_t)b * a.E + e] = run;
        run += cnt[(int64_t)b * a.E + e];
      }
    }
    carry += all;
    __syncthreads();  // sSeg and sBuf are reused by the next pass
  }
  if (tid == 0) a.offsets[a.E] = carry;
}

template <int PL>
__global__ __launch_bounds__(rp_threads<PL>()) void route_permute_kernel(RPArgs a) {
  constexpr int NT = rp_threads<PL>();
  constexpr int kTokPerWave = kRPBlock / (NT / 64);
  extern __shared__ int lds[];  // routing: hist [E] then bit rows [E][2]; scan: [NT] x 2
  __shared__ int sWord;
  const int tid = threadIdx.x;
  if (tid == 0) sWord = atomicAdd(&a.state->ticket, 1);
  __syncthreads();
  const int ticket = sWord;
  __syncthreads();

  if (a.T == 0) {  // one workgroup: zero offsets, header back to zero
    for (int e = tid; e <= a.E; e += NT) a.offsets[e] = 0;
    if (tid == 0) rp_reset(a.state);
    return;
  }
  if (ticket < a.nA) {
    // ---- routing block b ----
    const int b = ticket;
    int* hist = lds;
    uint32_t* bits = reinterpret_cast<uint32_t*>(lds + a.E);
    for (int i = tid; i < 3 * a.E; i += NT) lds[i] = 0;
    __syncthreads();
    const int wave = tid >> 6;
#pragma unroll 1
    for (int j = 0; j < kTokPerWave; ++j) {
      const int tl = wave * kTokPerWave + j;
      const int t = b * kRPBlock + tl;
      if (t < a.T) {
        auto pick = [&](int, int e) {
          atomicAdd(&hist[e], 1);
          atomicOr(&bits[2 * e + (tl >> 5)], 1u << (tl & 31));
        };
        if (a.mode == MOE_ROUTE_SIGMOID_BIAS)
          route_sigmoid_token<PL>(a.logits + (int64_t)t * a.E, a.bias, a.E, a.K, a.normalize,
                                  a.idx + (int64_t)t * a.K, a.gate + (int64_t)t * a.K, pick);
        else
          route_grouped_token<PL>(a.logits + (int64_t)t * a.E, a.E, a.G, a.Kp, a.idx + (int64_t)t * a.K,
                                  a.gate + (int64_t)t * a.K, pick);
      }
    }
    __syncthreads();  // histogram, bit rows and this block's selections complete
    for (int e = tid; e < a.E; e += NT) a.cnt[(int64_t)b * a.E + e] = hist[e];
    const int npairs = min(kRPBlock, a.T - b * kRPBlock) * a.K;
    for (int p = tid; p < npairs; p += NT) {
      const int tl = p / a.K;
      const int64_t j = (int64_t)(b * kRPBlock + tl) * a.K + p % a.K;
      const int e = a.idx[j];
      const uint32_t lo = bits[2 * e], hi = bits[2 * e + 1];
      const int rank = tl < 32 ? __popc(lo & ((1u << tl) - 1u)) : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
      a.dst_row[j] = rank;  // completed by the ranking phase
    }
    __threadfence();  // release this block's selections, counts and ranks
    __syncthreads();
    if (tid == 0) sWord = atomicAdd(&a.state->a_done, 1) == a.nA - 1;
    __syncthreads();
    if (!sWord) return;
    // ---- the last routing block: scan ----
    __threadfence();  // acquire every block's counts
    rp_scan<NT>(a, lds, lds + NT);
    __threadfence();  // release offsets and base rows
    __syncthreads();
    if (tid == 0) {
      if (a.nC == 0) rp_reset(a.state);
      else __hip_atomic_store(&a.state->ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (ticket >= a.nA + a.nC) {  // only with a header that was not zero
    if (tid == 0) atomicAdd(&a.state->timeouts, 1);
    return;
  }

  // ---- ranking of tokens [c * 512, c * 512 + 512) ----
  const int c = ticket - a.nA;
  if (tid == 0) {
    int ok = 0;
    for (int i = 0; i < kRPSpinLimit; ++i) {
      if (__hip_atomic_load(&a.state->ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) atomicAdd(&a.state->timeouts, 1);
    sWord = ok;
  }
  __syncthreads();
  if (sWord) {
    __threadfence();  // acquire the selections, ranks and base rows
    const int t0 = c * kRPRankTokens;
    const int npairs = min(kRPRankTokens, a.T - t0) * a.K;
    const int rows = a.T * a.K;
    for (int p = tid; p < npairs; p += NT) {
      const int t = t0 + p / a.K;
      const int64_t j = (int64_t)t0 * a.K + p;
      const int e = a.idx[j];
      const int d = a.base[(int64_t)(t / kRPBlock) * a.E + e] + a.dst_row[j];
      a.dst_row[j] = d;
      if (d >= 0 && d < rows) a.src_token[d] = t;  // always true with a zeroed header
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0 && atomicAdd(&a.state->c_done, 1) == a.nC - 1) rp_reset(a.state);
}

template <int PL>
struct LaunchRoutePermute {
  static void run(const RPArgs& a, hipStream_t st) {
    // routing: histogram + bit rows (3 E ints); scan: two NT-int arrays
    constexpr int NT = rp_threads<PL>();
    const size_t need = (size_t)3 * a.E * sizeof(int);
    const size_t lds = need > 2 * NT * sizeof(int) ? need : 2 * NT * sizeof(int);
    route_permute_kernel<PL><<<(unsigned)(a.nA + a.nC), NT, lds, st>>>(a);
  }
};

}  // namespace
}  // namespace moefp8

using namespace moefp8;

extern "C" moe_status moe_route_permute_workspace_size(int32_t T, int32_t K, int32_t E, size_t* bytes) {
  clear_detail();
  MOE_REQUIRE(bytes, MOE_ERR_NULL, "bytes is required");
  MOE_REQUIRE(T >= 0 && K >= 1 && E >= 1 && K <= E, MOE_ERR_SHAPE, "T=%d K=%d E=%d", T, K, E);
  MOE_REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "E=%d > 1024", E);
  const size_t nA = ((size_t)T + kRPBlock - 1) / kRPBlock;
  *bytes = kRPHeaderBytes + 2 * nA * (size_t)E * sizeof(int32_t);
  return MOE_OK;
}

extern "C" moe_status moe_route_permute(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K,
                                        int32_t n_groups, int32_t k_per_group, moe_route_mode mode,
                                        int32_t normalize_topk, int32_t* topk_idx, float* topk_gate,
                                        int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_detail();
  MOE_REQUIRE(mode == MOE_ROUTE_SIGMOID_BIAS || mode == MOE_ROUTE_SOFTMAX_GROUPED, MOE_ERR_UNSUPPORTED,
              "unknown route mode %d", (int)mode);
  MOE_REQUIRE(T >= 0 && E >= 1, MOE_ERR_SHAPE, "T=%d E=%d", T, E);
  MOE_REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "E=%d > 1024", E);
  MOE_REQUIRE(K >= 1 && K <= E, MOE_ERR_SHAPE, "need 1 <= K <= E (K=%d, E=%d)", K, E);
  if (mode == MOE_ROUTE_SOFTMAX_GROUPED) {
    MOE_REQUIRE(n_groups >= 1 && E % n_groups == 0, MOE_ERR_SHAPE, "E=%d not divisible by n_groups=%d", E,
                n_groups);
    MOE_REQUIRE(k_per_group >= 1 && k_per_group <= E / n_groups, MOE_ERR_SHAPE,
                "need 1 <= k_per_group <= E/n_groups (k_per_group=%d)", k_per_group);
    MOE_REQUIRE(K == n_groups * k_per_group, MOE_ERR_SHAPE, "K=%d != n_groups*k_per_group=%d", K,
                n_groups * k_per_group);
    MOE_REQUIRE(normalize_topk == 0, MOE_ERR_UNSUPPORTED, "grouped softmax gates are not renormalised");
  }
  MOE_REQUIRE((int64_t)T * K < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*K too large");
  MOE_REQUIRE(expert_offsets && workspace, MOE_ERR_NULL, "expert_offsets and workspace are required");
  MOE_REQUIRE(T == 0 || (logits && topk_idx && topk_gate && dst_row && src_token), MOE_ERR_NULL,
              "logits, topk_idx, topk_gate, dst_row and src_token are required");
  MOE_REQUIRE(aligned(logits, 4) && aligned(bias, 4) && aligned(topk_idx, 4) && aligned(topk_gate, 4) &&
                  aligned(expert_offsets, 4) && aligned(dst_row, 4) && aligned(src_token, 4),
              MOE_ERR_ALIGN, "4-byte alignment required");
  MOE_REQUIRE(aligned(workspace, 16), MOE_ERR_ALIGN, "workspace needs 16-byte alignment");
  size_t need = 0;
  moe_route_permute_workspace_size(T, K, E, &need);
  MOE_REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);

  RPArgs a;
  a.logits = logits;
  a.bias = mode == MOE_ROUTE_SIGMOID_BIAS ? bias : nullptr;
  a.T = T;
  a.E = E;
  a.K = K;
  a.G = mode == MOE_ROUTE_SOFTMAX_GROUPED ? n_groups : 1;
  a.Kp = mode == MOE_ROUTE_SOFTMAX_GROUPED ? k_per_group : K;
  a.mode = (int)mode;
  a.normalize = normalize_topk;
  a.idx = topk_idx;
  a.gate = topk_gate;
  a.offsets = expert_offsets;
  a.dst_row = dst_row;
  a.src_token = src_token;
  a.state = reinterpret_cast<RPState*>(workspace);
  const int nblk = (int)(((int64_t)T + kRPBlock - 1) / kRPBlock);
  a.cnt = reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) + kRPHeaderBytes);
  a.base = a.cnt + (size_t)nblk * E;
  a.nA = T == 0 ? 1 : nblk;  // T == 0: one workgroup writes the zero offsets
  a.nC = (int)(((int64_t)T + kRPRankTokens - 1) / kRPRankTokens);
  a.Ep = 1;
  while (a.Ep < E) a.Ep <<= 1;
  hipStream_t st = as_stream(stream);
  dispatch_per_lane<LaunchRoutePermute>(E, a, st);
  return after_launch("moe_route_permute", st);
}
