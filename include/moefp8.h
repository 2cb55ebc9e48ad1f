/*
 * moefp8.h -- C ABI of libmoefp8.so, the MI355X (gfx950) routed-expert FP8
 * MoE FFN layer.
 *
 * The operations follow three public write-ups:
 *   [KANANA-FP8] "Kakao Kanana-2 pre-training deep dive" (devday.kr), the
 *                paragraph on FP8 Tensor-Core training with fine-grained
 *                scaling, an all-experts MoE quantisation kernel and a
 *                transpose kernel for block-quantised weights;
 *   [DSV3-MOE]   "DeepSeek-V3 technical report summary" (theinnovators.zone),
 *                section 2.1, DeepSeekMoE bullets (shared + routed experts,
 *                sigmoid affinity then top-K, per-expert balancing bias, no
 *                token dropping);
 *   [DSV3-FP8]   same page, section 2.2, FP8 mixed-precision bullets (FP8
 *                GEMMs, 1x128 / 128x128 quantisation, promoted accumulation);
 *   [PANGU-MOGE] "Huawei releases open-weight models trained on Ascend"
 *                (amuse.peoplentools.com), Mixture-of-Grouped-Experts section
 *                (equal groups, K' picks per group, one global softmax,
 *                unselected scores 0, Imbalance Score 0).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every buffer argument is a DEVICE pointer (memory of the current HIP
 *    device).  Scalars are passed by value.  Row-major layouts throughout.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; no entry point synchronises the host.
 *  - The caller allocates and owns every buffer (including workspaces).  The
 *    library keeps no pointer after returning; enqueued kernels read and
 *    write the buffers until the stream reaches them.  No entry point
 *    allocates device memory.
 *  - Arguments are checked before anything is enqueued; on any error the
 *    function returns a non-zero status and launches nothing.  Checks never
 *    touch the device, so they also run on a host without a GPU.
 *  - A failed launch returns MOE_ERR_HIP; moe_last_error_detail() gives the
 *    HIP error text.  Device faults surface at the caller's next
 *    synchronisation.  With the environment variable MOEFP8_SYNC_CHECK=1
 *    every entry point synchronises its stream and reports device errors.
 *  - Preconditions that are NOT checked (undefined results if violated):
 *    finite inputs; expert ids in [0, E) and distinct within a token;
 *    group offsets non-decreasing with offsets[0] == 0 and offsets[G] == M.
 *  - FP8 codes are OCP E4M3FN bytes (bias 7, 3 mantissa bits, max 448, no
 *    infinities).  Quantisation: amax = max |x| over the tile or block,
 *    s = fl32(amax / 448) (s = 1 when amax == 0), code =
 *    RNE_E4M3(clamp(fl32(x / s), -448, 448)) with the sign kept; the value a
 *    code stands for is decode(code) * s.
 *  - Pointers to 16-byte vectors (codes, bf16 rows, fp32 rows) must be
 *    16-byte aligned (MOE_ERR_ALIGN otherwise); index and scale arrays need
 *    4-byte alignment.
 *  - Operands of more than 2^40 elements (beyond any device memory) are
 *    refused with MOE_ERR_UNSUPPORTED, before any size arithmetic.
 */
#ifndef MOEFP8_H
#define MOEFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                    */
  MOE_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, */
                           /* not a multiple of 128, or inconsistent        */
  MOE_ERR_UNSUPPORTED = 3, /* valid request outside what is implemented    */
  MOE_ERR_ALIGN = 4,       /* a pointer is not aligned as required          */
  MOE_ERR_WORKSPACE = 5,   /* the workspace is smaller than required        */
  MOE_ERR_HIP = 6          /* the HIP runtime reported an error             */
};

/* Element type and routing mode selectors are plain 32-bit integers (with
 * named values) rather than C enum types, so any value a caller passes is
 * well defined on the library side and an unknown one is refused with
 * MOE_ERR_UNSUPPORTED. */
typedef int32_t moe_dtype;
enum { MOE_F32 = 0, MOE_BF16 = 1 };

typedef int32_t moe_route_mode;
enum {
  MOE_ROUTE_SIGMOID_BIAS = 0,   /* [DSV3-MOE]   */
  MOE_ROUTE_SOFTMAX_GROUPED = 1 /* [PANGU-MOGE] */
};

/* Text of a status code (static storage). */
MOE_API const char* moe_status_string(moe_status s);
/* Detail of the last error on the calling thread (thread-local storage,
 * valid until the thread's next call into the library). */
MOE_API const char* moe_last_error_detail(void);

/*
 * moe_route -- token -> expert selection.            [DSV3-MOE], [PANGU-MOGE]
 *
 *  logits     f32 [T, E]   router scores (from moe_router_logits or the
 *                          caller's own projection)
 *  bias       f32 [E] or NULL (= zeros); SIGMOID_BIAS only
 *  T >= 0, 1 <= E <= 1024
 *  SIGMOID_BIAS: 1 <= K <= E; n_groups and k_per_group are ignored.
 *     s_e = sigmoid(l_e) (binary32 specification: 1 / (1 + E(-x)) with the
 *     Cody-Waite + degree-7 Taylor exp written out in the library source);
 *     key_e = fl32(s_e + bias_e); the K largest keys win, equal keys go to
 *     the lower expert index; slot k holds the k-th largest key.
 *     gate = s_e (the bias selects but does not weight); if normalize_topk,
 *     gate_k = fl32(s_k / S) with S summed in slot order in binary32.
 *  SOFTMAX_GROUPED: E % n_groups == 0, 1 <= k_per_group <= E / n_groups,
 *     K == n_groups * k_per_group.  Within each group the k_per_group
 *     largest logits win (equal logits -> lower index); slots are group-major,
 *     largest first.  gate = softmax over all E experts (computed in float64,
 *     rounded to float32), not renormalised; normalize_topk must be 0.
 *  topk_idx   i32 [T, K]   (out)
 *  topk_gate  f32 [T, K]   (out)
 * Errors: NULL logits/outputs -> MOE_ERR_NULL; bad sizes -> MOE_ERR_SHAPE;
 *         E > 1024 -> MOE_ERR_UNSUPPORTED.
 */
MOE_API moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K,
                     int32_t n_groups, int32_t k_per_group, moe_route_mode mode,
                     int32_t normalize_topk, int32_t* topk_idx, float* topk_gate, void* stream);

/*
 * moe_sigmoid_f32 -- y = sigmoid(x) elementwise with the binary32 sigmoid
 * specification moe_route applies to the affinity scores (and SwiGLU to its
 * gate), so that specification can be checked input by input.   [DSV3-MOE]
 *
 *  x, y   f32 [n] (device; y may equal x), n >= 0 (n == 0 launches nothing).
 *  Every finite or infinite input is defined; NaN inputs give unspecified
 *  values.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n < 0), MOE_ERR_ALIGN (x, y 16-byte),
 *         MOE_ERR_UNSUPPORTED (n above 2^40).
 */
MOE_API moe_status moe_sigmoid_f32(const float* x, int64_t n, float* y, void* stream);

/*
 * moe_permute_workspace_size -- bytes of device workspace moe_permute needs
 * for (T, K, E).  Host-only; never touches the device.
 */
MOE_API moe_status moe_permute_workspace_size(int32_t T, int32_t K, int32_t E, size_t* bytes);

/*
 * moe_permute -- group (token, slot) pairs by expert.       [DSV3-MOE], [PANGU-MOGE]
 *
 * No token is dropped and there is no capacity limit or padding: expert e
 * owns rows [offsets[e], offsets[e+1]) of the permuted operand, in ascending
 * token order (a stable counting sort of (expert, token) pairs; the result
 * does not depend on thread scheduling).
 *
 *  topk_idx        i32 [T, K]  expert ids (distinct within a token)
 *  xq, xs          u8 [T, H], f32 [T, H/128]  quantised tokens, or both NULL
 *                  to compute only the index maps
 *  expert_offsets  i32 [E+1]   (out) offsets[0] = 0, offsets[E] = T*K
 *  dst_row         i32 [T, K]  (out) permuted row of pair (t, k)
 *  src_token       i32 [T*K]   (out) token of permuted row r
 *  aq, as          u8 [T*K, H], f32 [T*K, H/128] (out; NULL iff xq is NULL)
 *                  aq[dst_row[t,k]] = xq[t], as[dst_row[t,k]] = xs[t]
 *  workspace       >= moe_permute_workspace_size(T, K, E) bytes, 16-B aligned
 *  With T == 0 only expert_offsets (all zeros on return) and the workspace
 *  are used; the other arrays may be NULL.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H % 128, K > E, ...),
 *         MOE_ERR_UNSUPPORTED (E > 1024), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE.
 */
MOE_API moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E,
                       const uint8_t* xq, const float* xs, int32_t H,
                       int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                       uint8_t* aq, float* as, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * moe_permute_noalloc -- moe_permute without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, same
 * results, bit for bit, minus (workspace, workspace_bytes).
 *
 * The counting scratch lives in a static device array of the library
 * (4 MiB per GPU, held until the process ends); its address is looked up
 * once per device on the first call there.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or host
 * threads) race and must be serialised by the caller.  The kernels write
 * every scratch element before reading it, so a call needs no clearing and
 * nothing is allocated, freed or copied.
 *
 * Errors: as moe_permute; MOE_ERR_WORKSPACE when (T, K, E) needs more scratch
 *         than the array holds (moe_permute_workspace_size(T, K, E) above
 *         4 MiB, e.g. T > 524032 at E = 256); MOE_ERR_HIP if the scratch
 *         address cannot be obtained.
 */
MOE_API moe_status moe_permute_noalloc(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E,
                               const uint8_t* xq, const float* xs, int32_t H,
                               int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                               uint8_t* aq, float* as, void* stream);

/*
 * moe_route_permute_workspace_size -- bytes of device workspace
 * moe_route_permute needs for (T, K, E).  Host-only.
 */
MOE_API moe_status moe_route_permute_workspace_size(int32_t T, int32_t K, int32_t E, size_t* bytes);

/*
 * moe_route_permute -- moe_route and the index maps of moe_permute in one
 * launch.                      [DSV3-MOE], [PANGU-MOGE]; operator fusion of
 *                              the Pangu page's system optimisation section
 *
 * Arguments as moe_route (logits .. topk_gate) and moe_permute's index maps
 * (expert_offsets, dst_row, src_token); the results are identical, bit for
 * bit, to moe_route followed by moe_permute with xq == NULL.  The
 * permutation's counting runs inside the routing workgroups and the ranking
 * workgroups wait (bounded) for the last routing workgroup's scan, so no
 * host or stream synchronisation separates the stages.
 *
 *  workspace  >= moe_route_permute_workspace_size(T, K, E) bytes, 16-B
 *             aligned.  Its first 256 bytes are counters kept between calls:
 *             ZERO-FILL them before the first use (e.g. hipMemset once after
 *             allocation); every call that completes leaves them zero again,
 *             so one workspace serves calls of any shapes it is large enough
 *             for.  The rest is scratch, written before it is read.  Calls
 *             that share a workspace must not overlap (same stream, or
 *             serialised).  Word 4 (int32) counts ranking workgroups whose
 *             wait ran out (never, with zeroed counters; such a workgroup
 *             writes nothing); it is never cleared by the library.
 *  With T == 0 only expert_offsets (all zeros) and the workspace are used.
 * Errors: as moe_route and moe_permute (MOE_ERR_WORKSPACE when the workspace
 *         is too small).
 */
MOE_API moe_status moe_route_permute(const float* logits, const float* bias, int32_t T, int32_t E, int32_t K,
                             int32_t n_groups, int32_t k_per_group, moe_route_mode mode,
                             int32_t normalize_topk, int32_t* topk_idx, float* topk_gate,
                             int32_t* expert_offsets, int32_t* dst_row, int32_t* src_token,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * quant_act_1x128_e4m3 -- per-(row, 128-column tile) FP8 quantisation of
 * activations.                                        [KANANA-FP8], [DSV3-FP8]
 *
 *  x      f32 or bf16 [rows, cols], cols % 128 == 0 (tiles run along the row,
 *         the GEMM reduction dimension)
 *  q      u8  [rows, cols]      (out) E4M3FN codes
 *  scale  f32 [rows, cols/128]  (out)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN.
 */
MOE_API moe_status quant_act_1x128_e4m3(const void* x, moe_dtype x_dtype, int64_t rows, int32_t cols,
                                uint8_t* q, float* scale, void* stream);

/*
 * quant_weight_128x128_e4m3 -- per-128x128-block FP8 quantisation of all G
 * experts' weights in one launch.                     [KANANA-FP8], [DSV3-FP8]
 *
 *  w      f32 or bf16 [G, rows, cols], rows % 128 == cols % 128 == 0; blocks
 *         anchored at (0, 0)
 *  q      u8  [G, rows, cols]            (out)
 *  scale  f32 [G, rows/128, cols/128]    (out)
 *  G == 0 launches nothing.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED (dtype, 2^31 or
 *         more blocks), MOE_ERR_ALIGN.
 */
MOE_API moe_status quant_weight_128x128_e4m3(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows,
                                     int32_t cols, uint8_t* q, float* scale, void* stream);

/*
 * quant_weight_128x128_e4m3_t -- quant_weight_128x128_e4m3 that also writes
 * the block-transposed codes and scales in the same pass: bit-identical to
 * quant_weight_128x128_e4m3 followed by fp8_block_transpose of (q, scale),
 * without the second read of q (the backward's operand: only the forward
 * FP8 weights are kept and the backward transposes them).     [KANANA-FP8]
 *
 *  w, w_dtype, G, rows, cols, q, scale: as quant_weight_128x128_e4m3
 *  qt       u8  [G, cols, rows]          (out, required)
 *  scale_t  f32 [G, cols/128, rows/128]  (out, required)
 * Errors: as quant_weight_128x128_e4m3; NULL qt or scale_t -> MOE_ERR_NULL.
 */
MOE_API moe_status quant_weight_128x128_e4m3_t(const void* w, moe_dtype w_dtype, int32_t G, int32_t rows,
                                       int32_t cols, uint8_t* q, float* scale, uint8_t* qt, float* scale_t,
                                       void* stream);

/*
 * grouped_gemm_fp8_blockscaled -- per-group C = A . B_g^T with block-scaled
 * FP8 operands and promoted accumulation.                        [DSV3-FP8]
 *
 *   C[m, n] = sum_kb ( sum_{k in kb} qa[m,k] * qb_g[n,k] ) * sa[m,kb] * sb_g[n/128, kb]
 * for offsets[g] <= m < offsets[g+1]; kb runs over 128-wide chunks of K.
 * Each chunk's FP8 dot products come from the matrix cores; the chunk result
 * is scaled and added to a float32 running sum (one fused multiply-add per
 * output per chunk), in chunk order.
 *
 *  aq  u8 [M, K], as f32 [M, K/128]           activations, 1x128 tiles
 *  bq  u8 [G, N, K], bs f32 [G, N/128, K/128] weights ([out, in] per group)
 *  group_offsets i32 [G+1] (device)           offsets[G] == M
 *  c   f32 or bf16 [M, N] (out); bf16 output is the RNE rounding of the
 *      float32 result.  Rows of empty groups do not exist; every row of C is
 *      written.
 *  Sizes: M >= 0 (M == 0 launches nothing), 1 <= G <= 1024, N % 128 == 0,
 *  K % 128 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED (G > 1024, K >
 *         65536, c_dtype), MOE_ERR_ALIGN.
 */
MOE_API moe_status grouped_gemm_fp8_blockscaled(const uint8_t* aq, const float* as, const uint8_t* bq,
                                        const float* bs, const int32_t* group_offsets, int32_t G, int64_t M,
                                        int32_t N, int32_t K, void* c, moe_dtype c_dtype, void* stream);

/*
 * grouped_gemm_fp8_blockscaled_gather -- grouped_gemm_fp8_blockscaled whose
 * grouped operand is gathered by row: row m of A is row a_row[m] of aq / as
 * (the permutation's src_token turns the token-order codes into the
 * expert-grouped operand without writing a permuted copy; the tokens are
 * dispatched to their experts with nothing dropped).          [DSV3-MOE]
 *
 *  aq  u8 [a_rows, K], as f32 [a_rows, K/128]  token-order activations
 *  a_row  i32 [M] (device, required)   indices outside [0, a_rows) are
 *         clamped into it; a_rows >= 1 and a_rows * K <= 2^32
 *  bq, bs, group_offsets, G, M, N, K, c, c_dtype: as grouped_gemm_fp8_blockscaled
 *  (same values, bit for bit, as the ungathered call on the gathered copy).
 * Errors: as grouped_gemm_fp8_blockscaled; MOE_ERR_UNSUPPORTED for a
 *         gathered operand above 4 GiB.
 */
MOE_API moe_status grouped_gemm_fp8_blockscaled_gather(const uint8_t* aq, const float* as, const int32_t* a_row,
                                               int64_t a_rows, const uint8_t* bq, const float* bs,
                                               const int32_t* group_offsets, int32_t G, int64_t M, int32_t N,
                                               int32_t K, void* c, moe_dtype c_dtype, void* stream);

/*
 * grouped_gemm_fp8_swiglu -- the gate|up grouped GEMM with SwiGLU and 1x128
 * FP8 quantisation of the result fused into its epilogue.   [DSV3-FP8]
 *
 * Computes, per group, G1 = A . B_g^T exactly as grouped_gemm_fp8_blockscaled
 * with N = 2I (bit-identical float32 values), then h = silu(g) * u with
 * g = G1[:, :I], u = G1[:, I:], silu(x) = fl32(x * sigmoid(x)) with the
 * binary32 sigmoid specification of moe_route, and quantises h in 1x128 tiles
 * along I.  The float32 G1 is never written.
 *
 *  aq, as, a_row, a_rows: as for grouped_gemm_fp8_blockscaled_gather; a_row
 *         may be NULL (then aq / as have M rows and a_rows is ignored)
 *  bq  u8 [G, 2I, K]: rows [0, I) are the gate projection, [I, 2I) the up
 *  hq  u8 [M, I], hs f32 [M, I/128]   (out, in grouped row order)
 *  Sizes: I % 128 == 0, K % 128 == 0.
 * Errors: as grouped_gemm_fp8_blockscaled.
 */
MOE_API moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, const int32_t* a_row,
                                   int64_t a_rows, const uint8_t* bq, const float* bs,
                                   const int32_t* group_offsets, int32_t G, int64_t M, int32_t I,
                                   int32_t K, uint8_t* hq, float* hs, void* stream);

/*
 * swiglu -- standalone SwiGLU + 1x128 FP8 quantisation.           [DSV3-FP8]
 *
 *  gate_up  f32 [M, 2I]  (g = columns [0, I), u = columns [I, 2I))
 *  hq       u8  [M, I]      (out)  codes of h = fl32(silu(g) * u)
 *  hs       f32 [M, I/128]  (out)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (I % 128), MOE_ERR_ALIGN.
 */
MOE_API moe_status swiglu(const float* gate_up, int64_t M, int32_t I, uint8_t* hq, float* hs,
                  void* stream);

/*
 * moe_combine -- gate-weighted sum of each token's expert outputs plus the
 * shared expert's output, stored as bf16.                        [DSV3-MOE]
 *
 *   acc = 0; for k = 0..K-1: acc = fl32(acc + fl32(gate[t,k] * y_perm[dst_row[t,k], n]));
 *   acc = fl32(acc + shared[t, n]) (if shared != NULL); out[t, n] = bf16_rne(acc)
 *
 *  y_perm     f32 [T*K, H]  expert outputs in permuted order
 *  dst_row    i32 [T, K]    from moe_permute
 *  topk_gate  f32 [T, K]    from moe_route
 *  shared     f32 [T, H] or NULL
 *  out_bf16   u16 [T, H] (out) bf16 bit patterns
 *  H % 8 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN.
 */
MOE_API moe_status moe_combine(const float* y_perm, const int32_t* dst_row, const float* topk_gate,
                       const float* shared, int32_t T, int32_t K, int32_t H, uint16_t* out_bf16,
                       void* stream);

/*
 * grouped_gemm_fp8_combine_workspace_size -- bytes of the arrival counters
 * grouped_gemm_fp8_combine needs for T tokens and N output columns.
 * Host-only.
 */
MOE_API moe_status grouped_gemm_fp8_combine_workspace_size(int32_t T, int32_t N, size_t* bytes);

/*
 * grouped_gemm_fp8_combine -- the down projection with moe_combine fused into
 * its epilogue.            [DSV3-FP8], [DSV3-MOE]; operator fusion of the
 *                          Pangu page's system optimisation section
 *
 * Writes c exactly as grouped_gemm_fp8_blockscaled(aq, as, bq, bs,
 * group_offsets, G, M, N, K, c, MOE_F32) and y exactly as
 * moe_combine(c, dst_row, topk_gate, shared, T, topk, N, y_bf16), bit for
 * bit, in one launch: the workgroup tile that finishes last among the topk
 * tiles holding a token's rows (per 256-column slice; an arrival counter
 * elects it) sums them in slot order.  The election never changes the order
 * of the sum, so y does not depend on scheduling.
 *
 *  aq .. K, c   as grouped_gemm_fp8_blockscaled with c f32 [M, N] (out)
 *  src_token    i32 [M]        token of grouped row m       (moe_permute)
 *  dst_row      i32 [T, topk]  grouped row of (t, k)        (moe_permute)
 *  topk_gate    f32 [T, topk]                               (moe_route)
 *  shared       f32 [T, N] or NULL; must be complete when the launch starts
 *  y_bf16       u16 [T, N] (out) bf16 bit patterns
 *  counters     >= grouped_gemm_fp8_combine_workspace_size(T, N) bytes,
 *               ZERO-FILLED before the first use (e.g. hipMemset once after
 *               allocation); every call that completes leaves them zero.
 *               Calls sharing counters must not overlap.
 *  M == T * topk (no token dropped); src_token and dst_row must be a
 *  permutation and its inverse, as moe_permute writes them (otherwise y is
 *  unspecified and the counters may be left non-zero; no access leaves the
 *  buffers).
 * Errors: as grouped_gemm_fp8_blockscaled; MOE_ERR_SHAPE (M != T * topk),
 *         MOE_ERR_WORKSPACE (counters too small).
 */
MOE_API moe_status grouped_gemm_fp8_combine(const uint8_t* aq, const float* as, const uint8_t* bq,
                                    const float* bs, const int32_t* group_offsets, int32_t G, int64_t M,
                                    int32_t N, int32_t K, float* c, const int32_t* src_token,
                                    const int32_t* dst_row, const float* topk_gate, const float* shared,
                                    int32_t T, int32_t topk, uint16_t* y_bf16, int32_t* counters,
                                    size_t counters_bytes, void* stream);

/*
 * fp8_block_transpose -- transpose of block-quantised weights, codes and
 * scale grid, as exact bit copies (the backward pass's operand without
 * re-quantising).                                               [KANANA-FP8]
 *
 *  q        u8  [G, rows, cols],      scale   f32 [G, rows/128, cols/128]
 *  qt       u8  [G, cols, rows] (out), scale_t f32 [G, cols/128, rows/128] (out)
 *  rows % 128 == cols % 128 == 0.  q and qt must not overlap.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN.
 */
MOE_API moe_status fp8_block_transpose(const uint8_t* q, const float* scale, int32_t G, int32_t rows,
                               int32_t cols, uint8_t* qt, float* scale_t, void* stream);

/* ------------------------------------------------------------------------
 * Input-side backward.  [KANANA-FP8]: the backward expert GEMMs run in FP8
 * on the block-transposed forward weights (fp8_block_transpose, then
 * grouped_gemm_fp8_blockscaled with the transposed copy as B); their inputs
 * are quantised in 1x128 tiles along the reduction dimension ([DSV3-FP8]).
 * Gradients pass straight through the FP8 rounding.
 * ------------------------------------------------------------------------ */

/*
 * moe_combine_backward -- gradient of the gate-weighted combine
 * y[t] = sum_k gate[t,k] * y_perm[dst_row[t,k]] (+ shared[t]).   [DSV3-MOE]
 *
 *  dy        bf16 [T, H] (raw 16-bit patterns)  upstream gradient
 *  y_perm    f32  [T*K, H]   the forward's expert outputs (permuted order)
 *  dst_row   i32  [T, K], topk_gate f32 [T, K]  as in moe_combine
 *  dq, ds    u8 [T*K, H], f32 [T*K, H/128] (out): fl32(gate[t,k] * dy[t])
 *            written at row dst_row[t,k], quantised in 1x128 tiles (the FP8
 *            operand of the down projection's dgrad)
 *  d_gate    f32  [T, K] (out): <dy[t], y_perm[dst_row[t,k]]>, summed in a
 *            fixed order (reproducible)
 *  gate_row  f32  [T*K] (out, optional, NULL to skip): gate_row[dst_row[t,k]]
 *            = topk_gate[t,k], the gate of each grouped row (the row factor
 *            of the down projection's weight-gradient operand)
 *  The shared expert's gradient is dy itself (quantise it with
 *  quant_act_1x128_e4m3).  H % 128 == 0, 1 <= K <= 16.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED (K > 16), MOE_ERR_ALIGN
 *         (dy, y_perm 16-byte; dq 8-byte).
 */
MOE_API moe_status moe_combine_backward(const uint16_t* dy_bf16, const float* y_perm, const int32_t* dst_row,
                                const float* topk_gate, int32_t T, int32_t K, int32_t H, uint8_t* dq,
                                float* ds, float* d_gate, float* gate_row, void* stream);

/*
 * swiglu_backward -- gradient of h = silu(g) * u, [g | u] the float32
 * gate|up GEMM output, with the result quantised for the gate|up dgrad.
 *
 *  gate_up  f32 [M, 2I]  the forward's gate|up output (g = [:, :I], u = [:, I:])
 *  dh       f32 [M, I]   gradient of h
 *  dq, ds   u8 [M, 2I], f32 [M, 2I/128] (out): [dg | du] quantised in 1x128
 *           tiles, with (binary32, s the sigmoid specification of moe_route):
 *           silu = g*s; dsilu = s*(1 + g*(1 - s)); du = dh*silu; dg = (dh*u)*dsilu
 *  d        f32 [M, 2I] (out, optional, NULL to skip): [dg | du] unquantised
 *           (the source of the gate|up weight gradient's 128x1 operand)
 *  I % 128 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN (gate_up, dh 16-byte).
 */
MOE_API moe_status swiglu_backward(const float* gate_up, const float* dh, int64_t M, int32_t I, uint8_t* dq,
                           float* ds, float* d, void* stream);

/*
 * moe_route_backward -- gradient of the gates with respect to the router
 * logits, through the selected experts only (top-K selection is piecewise
 * constant; the balancing bias selects but does not weight).
 *                                                 [DSV3-MOE], [PANGU-MOGE]
 *  logits    f32 [T, E], topk_idx i32 [T, K]   the forward's inputs / selection
 *  d_gate    f32 [T, K]   gradient of the gates (moe_combine_backward)
 *  mode, normalize_topk   as in moe_route (n_groups is not needed)
 *  d_logits  f32 [T, E] (out), every element written:
 *    SIGMOID_BIAS: s_k = sigmoid(l_k); dL/ds_k = (d_gate_k - sum_j d_gate_j gate_j) / S
 *      with S = sum_j s_j when normalised (else d_gate_k); dL/dl = dL/ds_k s_k (1 - s_k)
 *      at the selected experts, 0 elsewhere.
 *    SOFTMAX_GROUPED: p = softmax(l) over all E, gate_k = p[topk_idx[k]];
 *      dL/dl_j = p_j (D_j - sum_k d_gate_k gate_k), D_j = d_gate_k at j = topk_idx[k].
 *  Evaluated in float64 and rounded once.  K <= 64; topk_idx values outside
 *  [0, E) contribute nothing.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN.
 */
MOE_API moe_status moe_route_backward(const float* logits, const int32_t* topk_idx, const float* d_gate,
                              int32_t T, int32_t E, int32_t K, moe_route_mode mode, int32_t normalize_topk,
                              float* d_logits, void* stream);

/* ------------------------------------------------------------------------
 * Weight gradients of the expert GEMMs in FP8.  [DSV3-FP8]: most training
 * GEMMs, backward ones included, run in FP8 with fine-grained scaling.  For
 * a projection out = in . W_g^T (W_g stored [out, in]) of expert g:
 *   dW_g[o, i] = sum over the expert's rows r of dOut[r, o] * In[r, i],
 * a reduction over tokens.  Both operands are quantised in 128x1 tiles
 * (128 consecutive rows of one expert in one column; each expert's rows are
 * padded with zero rows to whole tiles so no tile spans two experts; scale
 * and codes as in the conventions above) and stored transposed, [column,
 * padded row] with row stride ld, expert g owning the padded rows
 * [P_g, P_{g+1}), P_g = sum over g' < g of 128 ceil(M_g' / 128).
 * ------------------------------------------------------------------------ */

/*
 * moe_wgrad_padded_rows -- host-only: the smallest admissible ld for M
 * grouped rows in G groups, 128 (ceil(M/128) + G) (an upper bound on P_G).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE.
 */
MOE_API moe_status moe_wgrad_padded_rows(int64_t M, int32_t G, int64_t* rows);

/*
 * quant_act_128x1_grouped_e4m3 -- 128x1-tile quantisation of a grouped
 * operand, written transposed.
 *
 *  x            [x_rows, C] (f32 or bf16), or with swiglu_input != 0 a float32
 *               gate|up array [x_rows, 2C] whose rows give h = silu(g) * u
 *               (the forward's binary32 SwiGLU, g = [:, :C], u = [:, C:])
 *  row_index    i32 [M] or NULL: grouped row r reads row row_index[r] of x
 *               (indices clamped into [0, x_rows)); NULL reads row r
 *  row_scale    f32 [M] or NULL: grouped row r is fl32(row_scale[r] * value)
 *  group_offsets i32 [G+1] (device): grouped rows of expert g are
 *               [offsets[g], offsets[g+1]); offsets[G] == M
 *  ld           row stride of qt (multiple of 128, >= moe_wgrad_padded_rows)
 *  padded_offsets i32 [G+1] (out): P_0..P_G
 *  qt           u8  [C, ld] (out): codes; columns [P_g, P_{g+1}) hold expert
 *               g's rows then zero codes for its padding rows; columns past
 *               P_G are not written
 *  st           f32 [ld/128, C] (out): tile scales, tile-major (tile j of
 *               column c at st[j, c], for the tiles below P_G)
 *  C % 128 == 0, 1 <= G <= 1024.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (C, ld, x_rows), MOE_ERR_UNSUPPORTED
 *         (dtype, G, a bf16 gate|up input, more than 2^31 - 1 blocks of 128
 *         rows x 64 columns), MOE_ERR_ALIGN (x, qt 16-byte).
 */
MOE_API moe_status quant_act_128x1_grouped_e4m3(const void* x, moe_dtype x_dtype, int32_t swiglu_input,
                                        int64_t x_rows, int32_t C, const int32_t* row_index,
                                        const float* row_scale, const int32_t* group_offsets, int32_t G,
                                        int64_t M, int64_t ld, int32_t* padded_offsets, uint8_t* qt,
                                        float* st, void* stream);

/*
 * grouped_wgrad_fp8 -- dW_g = A_g . B_g^T over expert g's padded rows,
 * promoted per 128-row chunk:
 *   dW_g[o, i] = sum_kb P_kb[o, i] * as[kb, o] * bs[kb, i]
 * with P_kb the FP8 dot product of the chunk (float32 accumulation).
 *
 *  aq, as   u8 [Na, ld], f32 [ld/128, Na]   output-gradient operand (dOut^T)
 *  bq, bs   u8 [Nb, ld], f32 [ld/128, Nb]   input operand (In^T)
 *  padded_offsets i32 [G+1] (device)   from quant_act_128x1_grouped_e4m3
 *  c        [G, Na, Nb] (out), f32 or bf16 (RNE): the [out, in] layout of the
 *           weights; an expert without rows gets zeros.  accumulate != 0
 *           adds to c's contents instead (c = c + dW in float32, then the
 *           output type's rounding).
 *  Na % 128 == Nb % 128 == 0, 1 <= G <= 1024, ld a multiple of 128 and at
 *  most 2^29.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED (dtype, G, ld above
 *         2^29, more than 2^31 - 8 output tiles of 256 x 256), MOE_ERR_ALIGN
 *         (aq, bq 16-byte; c 16-byte for f32, 8-byte for bf16; a bf16 c
 *         that is 16-byte aligned is written with 16-byte stores, faster,
 *         with the same values).
 */
MOE_API moe_status grouped_wgrad_fp8(const uint8_t* aq, const float* as, const uint8_t* bq, const float* bs,
                             const int32_t* padded_offsets, int32_t G, int32_t Na, int32_t Nb, int64_t ld,
                             void* c, moe_dtype c_dtype, int32_t accumulate, void* stream);

/* ------------------------------------------------------------------------
 * Router projection and the balancing bias.  [DSV3-MOE]: affinity scores
 * come from the router; a per-expert bias, adjusted to balance the load
 * instead of an auxiliary loss, shifts the top-K selection (see moe_route).
 * ------------------------------------------------------------------------ */

/*
 * moe_router_logits -- logits = x . W_r^T in float32 (the gating path is not
 * quantised): logits[t, e] = sum_h x[t, h] * w_router[e, h], float32 products
 * and sums on the matrix cores (summation order unspecified; error within
 * (H + 2) 2^-24 sum_h |x w| of the exact sum).
 *
 *  x_bf16    bf16 [T, H] (raw 16-bit patterns)   layer input
 *  w_router  f32  [E, H]                          router weight
 *  logits    f32  [T, E] (out)                    input of moe_route
 *  T >= 0 (T == 0 launches nothing), H % 64 == 0, 1 <= E <= 4194240.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN
 *         (x_bf16, w_router 16-byte).
 */
MOE_API moe_status moe_router_logits(const uint16_t* x_bf16, const float* w_router, int32_t T, int32_t H,
                             int32_t E, float* logits, void* stream);

/*
 * moe_bias_update -- one step of the aux-loss-free balancing (a reading: the
 * pages do not give the rule): with load_e = offsets[e+1] - offsets[e] (the
 * step's grouped rows per expert, moe_permute's offsets) and the mean load
 * (offsets[E] - offsets[0]) / E,
 *   bias[e] = fl32(bias[e] - gamma * sign(load_e - mean)),
 * the sign decided exactly on integers.
 *
 *  expert_offsets i32 [E+1] (device), gamma (by value), bias f32 [E] (in/out).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN.
 */
MOE_API moe_status moe_bias_update(const int32_t* expert_offsets, int32_t E, float gamma, float* bias,
                           void* stream);

/*
 * moe_probe_mfma_fp8 -- measurement helper, not a step of the layer: the
 * FP8 matrix cores' own ceiling on this device (the figure the grouped
 * GEMMs' rates are read against beside the datasheet peak).  `blocks`
 * workgroups of `waves_per_block` waves each run 8 independent chains of
 * `iters` V_MFMA_SCALE_F32_16X16X128_F8F6F4 on register operands whose every
 * E4M3 code is `code`; each lane then writes the sum of its accumulators to
 * out[64 * waves_per_block * block + lane] (so for a code of value v that sum
 * is exactly 4096 v^2 iters while it stays an integer below 2^24), and
 * *flops (host) receives the launch's flop count, 8 * 65536 per wave and
 * iteration.  Time it with events on `stream`.
 *
 *  out f32 [blocks * 64 * waves_per_block] (device, written), flops (host).
 *  0 <= iters <= 2^32, 1 <= blocks <= 2^20, 1 <= waves_per_block <= 16.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN (out 4-byte).
 */
MOE_API moe_status moe_probe_mfma_fp8(uint8_t code, int64_t iters, int32_t blocks, int32_t waves_per_block,
                                      float* out, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEFP8_H */
