/*
 * moe.h — C ABI of libmoe.so: the forward pass of one DeepSeek-V3 MoE layer on
 * one AMD Instinct MI355X (gfx950).
 *
 * The layer (sources are the pages about the DeepSeek-V3 technical report):
 *   route    sigmoid token-to-expert affinity, a per-expert bias used only for
 *            selection, group-limited top-k, gates normalised over the selected
 *            set and scaled ("DeepSeek-V3" summary page, section 1 DeepSeekMoE
 *            and node-limited routing, section 2 auxiliary-loss-free balancing;
 *            the book's chapters 7 and 8)
 *   quant    FP8 E4M3 with one FP32 scale per 1x128 activation tile or per
 *            128x128 weight block, scale = amax/448 from the current tile
 *            (summary page section 6 (a), (c), (d); book chapter 16)
 *   permute  group the (token, expert) assignments by expert, keeping the
 *            source token of every row (book chapter 15 "What dispatch must do")
 *   gemm     SwiGLU experts as a ragged grouped FP8 GEMM whose 128-wide K-block
 *            partial sums are promoted to FP32 with the block scales applied
 *            (summary page section 6 (b); book chapter 16 "Periodic
 *            high-precision promotion"), the intermediate requantised 1x128
 *            (book chapter 17 "SwiGLU recomputation"), BF16 output
 *   combine  gated sum of each token's routed expert outputs plus the shared
 *            expert, in BF16 (book chapter 7, chapter 15 "What combine must do",
 *            chapter 17 "FP8 dispatch, BF16 combine")
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers, allocated and owned by the caller.  The
 *     library never allocates, frees or synchronises; every call is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream) and
 *     returns after host-side validation and launch.
 *   - Row-major layouts, last dimension contiguous.  BF16 is passed as uint16_t
 *     bit patterns, E4M3 codes as uint8_t.
 *   - Byte (E4M3, uint8) and BF16 matrices must be 16-byte aligned; FP32 and
 *     int32 arrays 4-byte aligned.
 *   - Return MOE_OK, or an error code with no work enqueued; moe_last_error()
 *     then describes the failure (thread-local).  An asynchronous kernel fault
 *     shows up at the caller's next synchronisation, not here.
 *   - T = 0 (no tokens) is a successful no-op.
 *   - Shapes: d % 128 == 0, f % 128 == 0, 1 <= E <= 256, E % G == 0,
 *     1 <= M <= G <= 64, k % M == 0, 1 <= k <= min(16, M*E/G), k/M <= E/G.
 *   - NaN or Inf inputs are outside the contract.
 *   - The shared expert is group index E of the grouped GEMM; it owns rows
 *     [T*k, T*k + T) of the permuted order, in token order, with weight 1.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad shape or parameter, misalignment */
  MOE_ERR_UNSUPPORTED = 2,  /* valid request beyond what the kernels implement */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  MOE_ERR_HIP = 4           /* a HIP launch error */
} moe_status;

/* Routing parameters.  V3: n_experts 256, n_groups 8, topk_groups 4, topk 8,
 * route_scale 2.5 (the routed scaling factor of the released configuration,
 * applied after normalisation: book chapter 7). */
typedef struct {
  int n_experts;    /* E: routed experts; expert e belongs to group e / (E/G) */
  int n_groups;     /* G: groups (nodes in the report's terms) */
  int topk_groups;  /* M: groups a token may use */
  int topk;         /* k (K_r): routed experts per token */
  float route_scale;
} moe_route_params;

/* moe_route — router of one MoE layer (summary page section 1; book chapters 7-8).
 *   x       [T, d] BF16 token inputs u_t
 *   wg      [E, d] BF16 expert centroids e_i
 *   bias    [E] FP32 selection bias b_i, or NULL for zero
 *   idx     [T, k] int32 out: selected experts in ascending id
 *   w       [T, k] FP32 out: route_scale * s_i / sum of s over the selected set
 * Affinity s = sigmoid(u . e) (FP32 products accumulated per 128-wide K block,
 * blocks summed in FP64); selection score z = s + b; group score = sum of the
 * k/M largest z in the group; the M best groups are kept (ties to the lower
 * group index); the k largest z among their experts are selected (ties to the
 * lower expert index).  The selection ranks FP32 biased scores: the logit
 * rounded to FP32, an FP32 sigmoid (exp and the hardware reciprocal, a few
 * ulp from exact), plus the bias; ranks move only within 1e-6 near ties.
 * The gates are evaluated in FP64 and rounded to FP32. */
moe_status moe_route(const uint16_t* x, const uint16_t* wg, const float* bias,
                     int T, int d, moe_route_params p,
                     int32_t* idx, float* w, void* stream);

/* Bytes of device workspace moe_route_ws needs for T tokens and E experts
 * (FP32 logits [T, E], rounded up to 256), or 0 where it uses moe_route's
 * single kernel (T above 8192, or T, E out of range). */
size_t moe_route_workspace_bytes(int T, int E);

/* moe_route_ws — moe_route with a caller-owned workspace, the same results
 * bit for bit.  For small batches one workgroup per 64 tokens would stream
 * all E centroid rows alone; here the logits are computed by workgroups of
 * (16 tokens, 32 experts) for T <= 1024 or (64 tokens, 64 experts) for
 * T <= 8192, each over all of d in the same order of arithmetic, written to
 * the workspace, and a second kernel selects.
 *   workspace        device memory of at least moe_route_workspace_bytes(T, E)
 *                    bytes, 4-byte aligned (may be NULL when that is 0);
 *                    overwritten; calls that share it must not overlap
 * Errors as moe_route, and MOE_ERR_WORKSPACE for a missing, misaligned or
 * short workspace. */
moe_status moe_route_ws(const uint16_t* x, const uint16_t* wg, const float* bias,
                        int T, int d, moe_route_params p, int32_t* idx, float* w,
                        void* workspace, size_t workspace_bytes, void* stream);

/* fp8_quant_1x128 — activation quantisation (summary page section 6 (a), (d)).
 *   x      [rows, cols] BF16, cols % 128 == 0
 *   q      [rows, cols] E4M3 out
 *   scale  [rows, cols/128] FP32 out: amax/448 of each 1x128 tile (1.0 if amax = 0)
 * q = E4M3(fl32(x / scale)), round to nearest even, saturating at +-448,
 * subnormals kept. */
moe_status fp8_quant_1x128(const uint16_t* x, int rows, int cols,
                           uint8_t* q, float* scale, void* stream);

/* fp8_quant_128x128 — weight quantisation, same rule per 128x128 block.
 *   w      [N, K] BF16, N % 128 == 0, K % 128 == 0 (a stack of matrices whose
 *          row counts are multiples of 128 may be passed as one [N, K])
 *   q      [N, K] E4M3 out
 *   scale  [N/128, K/128] FP32 out (the dequantisation multiplier) */
moe_status fp8_quant_128x128(const uint16_t* w, int N, int K,
                             uint8_t* q, float* scale, void* stream);

/* Bytes of device workspace moe_permute needs for T tokens, k slots, E experts. */
size_t moe_permute_workspace_bytes(int T, int k, int E);

/* moe_permute — group assignments by expert (book chapters 7 and 15).
 *   idx        [T, k] int32 selected experts (distinct per token, in [0, E))
 *   offsets    [E+2] int32 out: expert e owns rows [offsets[e], offsets[e+1]);
 *              offsets[E] = T*k, offsets[E+1] = T*k + T (shared expert)
 *   pos        [T, k] int32 out: row of assignment (t, idx[t][j])
 *   row_token  [T*k + T] int32 out: source token of every row (the shared
 *              rows are the identity)
 *   xq, xs     [T, d] E4M3 and [T, d/128] FP32 quantised inputs, or NULL
 *   xq_perm, xs_perm  [T*k + T, d] and [T*k + T, d/128] out: the rows copied
 *              into grouped order (the dispatch), or NULL to produce only the
 *              metadata (the grouped GEMM can gather through row_token)
 * Within an expert rows follow token order, so the result is unique.  Integer
 * work only, deterministic (no order-dependent atomics). */
moe_status moe_permute(const int32_t* idx, int T, int k, int E,
                       const uint8_t* xq, const float* xs, int d,
                       int32_t* offsets, int32_t* pos, int32_t* row_token,
                       uint8_t* xq_perm, float* xs_perm,
                       void* workspace, size_t workspace_bytes, void* stream);

/* moe_permute_noalloc — moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results bit for bit, without the
 * workspace.  Its per-block histograms live in a static device array of the
 * library, 1 MiB per GPU (held until the process ends), so
 * ceil(T/256) * E <= 262144 (T <= 262144 tokens at E = 256); larger calls
 * return MOE_ERR_UNSUPPORTED.  Allocates nothing (no hipMalloc, hipFree or
 * allocating library call).  Calls on one GPU share the array: calls that
 * overlap in time on one GPU (concurrent streams, several host threads) race
 * and must be serialised by the caller.  Errors as moe_permute, plus
 * MOE_ERR_HIP if the array's device address cannot be obtained on the
 * current device. */
moe_status moe_permute_noalloc(const int32_t* idx, int T, int k, int E,
                               const uint8_t* xq, const float* xs, int d,
                               int32_t* offsets, int32_t* pos, int32_t* row_token,
                               uint8_t* xq_perm, float* xs_perm, void* stream);

/* grouped_gemm_fp8_swiglu — all experts of the layer (summary page section 6;
 * book chapters 7, 16, 17).  For every group g in [0, n_groups) (E routed
 * experts, then the shared expert) and every row r in [offsets[g], offsets[g+1]):
 *   a_r   = row row_src[r] of (aq, as)  (row r itself when row_src is NULL)
 *   G, U  = blocked FP8 GEMMs of a_r with W1 = w13[g][0:f] and W3 = w13[g][f:2f]:
 *           sum over 128-wide K blocks of (as * ws) * (exact block dot product),
 *           accumulated in FP32
 *   h     = SiLU(G) * U in FP32, quantised 1x128 -> h [rows, f] E4M3,
 *           hs [rows, f/128] FP32
 *   y     = blocked FP8 GEMM of h with w2[g] -> BF16 [rows, d]
 *   aq [a_rows, d] E4M3, as [a_rows, d/128] FP32
 *   row_src  [total_rows] int32 in [0, a_rows), or NULL
 *   offsets  [n_groups + 1] int32, non-decreasing, offsets[0] = 0,
 *            offsets[n_groups] = total_rows (moe_permute's array works)
 *   w13 [n_groups, 2f, d] E4M3, w13_s [n_groups, 2f/128, d/128] FP32
 *   w2  [n_groups, d, f]  E4M3, w2_s  [n_groups, d/128, f/128]  FP32
 *   h, hs, y  outputs as above (h/hs are also the input of the second GEMM)
 * Row counts per group are read on the device: nothing waits on the host.
 * MOE_ERR_UNSUPPORTED: n_groups > 1024, or 2f*d or total_rows*max(d, f) (or
 * a_rows*d) above 2^32 bytes (the kernels use 32-bit byte offsets). */
moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, int a_rows,
                                   const int32_t* row_src, const int32_t* offsets,
                                   int n_groups, int total_rows, int d, int f,
                                   const uint8_t* w13, const float* w13_s,
                                   const uint8_t* w2, const float* w2_s,
                                   uint8_t* h, float* hs, uint16_t* y, void* stream);

/* grouped_gemm_fp8_up — the first stage of grouped_gemm_fp8_swiglu alone:
 * G, U, h = SiLU(G) * U and its 1x128 quantisation into (h, hs), same
 * arguments and rules as above.  Separately callable so that the two expert
 * GEMMs can be scheduled, timed or recomputed on their own. */
moe_status grouped_gemm_fp8_up(const uint8_t* aq, const float* as, int a_rows,
                               const int32_t* row_src, const int32_t* offsets,
                               int n_groups, int total_rows, int d, int f,
                               const uint8_t* w13, const float* w13_s,
                               uint8_t* h, float* hs, void* stream);

/* grouped_gemm_fp8_down — the second stage alone: y = blocked FP8 GEMM of
 * (h, hs) [total_rows, f] with w2[g] per group, BF16 out [total_rows, d]. */
moe_status grouped_gemm_fp8_down(const uint8_t* h, const float* hs, const int32_t* offsets,
                                 int n_groups, int total_rows, int d, int f,
                                 const uint8_t* w2, const float* w2_s,
                                 uint16_t* y, void* stream);

/* moe_combine — out[t] = BF16( sum_j w[t][j] * y[pos[t][j]] + y[shared_row0 + t]
 *                              + residual[t] )
 * (book chapter 7 "Selecting and combining experts"; chapter 15 "What combine
 * must do", which lists the residual path among what combine adds), summed in
 * FP32 in slot order, then the shared row, then the residual, rounded once.
 *   y            [rows, d] BF16 expert outputs
 *   pos, w       [T, k] rows and gates of each token
 *   shared_row0  first shared-expert row (T*k), or -1 for none
 *   residual     [T, d] BF16, or NULL for none (the layer passes none: its
 *                output is the MoE branch)
 *   out          [T, d] BF16 (may not alias y or residual) */
moe_status moe_combine(const uint16_t* y, const int32_t* pos, const float* w,
                       int T, int k, int d, int32_t shared_row0,
                       const uint16_t* residual, uint16_t* out, void* stream);

/* moe_bias_update — one step of the auxiliary-loss-free balancing controller
 * ("DeepSeek-V3: the recipe, and the interconnect that shaped it", section
 * "Auxiliary-loss-free balancing"; summary page section 2; book chapter 8
 * "V3's routing-only bias"): for every routed expert e < n_experts,
 *   bias[e] -= gamma * sign(load[e] - mean load)
 * with load[e] = offsets[e+1] - offsets[e] (moe_permute's array) and the mean
 * taken over the n_experts routed experts (offsets[n_experts] assignments);
 * an expert exactly at the mean keeps its bias.  The comparison is exact
 * (integers), the update FP32 with one rounding.
 *   offsets  [n_experts + 1 or more] int32 on the device
 *   bias     [n_experts] FP32 on the device, updated in place
 * MOE_ERR_INVALID_ARG: n_experts < 1, gamma not finite, misaligned pointers. */
moe_status moe_bias_update(const int32_t* offsets, int n_experts, float gamma, float* bias,
                           void* stream);

/* ---- Power-of-two (E8M0) scale variant ----
 * The pages' training recipe uses power-of-two scaling factors for some
 * tensors (summary page section 6; book chapter 17), and block-scaled matrix
 * hardware takes one 8-bit exponent per block (summary page section 6,
 * microscaling).  In this variant every scale is the smallest power of two
 * not below fl32(amax/448), at least 2^-127, 1.0 for an all-zero tile; it is
 * stored as that FP32 value in the same arrays as above, so its FP32 exponent
 * field is its E8M0 code.  Codes are E4M3(fl32(x / scale)) as before.  With
 * such scales the GEMMs pass the scales to gfx950's block-scaled MFMA and
 * accumulate in the instruction (no software promotion). */

/* fp8_quant_1x128_pow2 / fp8_quant_128x128_pow2 — fp8_quant_1x128 and
 * fp8_quant_128x128 with the power-of-two scale rule; same arguments, layouts
 * and errors. */
moe_status fp8_quant_1x128_pow2(const uint16_t* x, int rows, int cols,
                                uint8_t* q, float* scale, void* stream);
moe_status fp8_quant_128x128_pow2(const uint16_t* w, int N, int K,
                                  uint8_t* q, float* scale, void* stream);

/* grouped_gemm_fp8_up_e8m0 / grouped_gemm_fp8_down_e8m0 — grouped_gemm_fp8_up
 * and grouped_gemm_fp8_down for operands whose every scale (as, w13_s, hs,
 * w2_s) is a power of two in [2^-127, 2^127], as the _pow2 quantisers write
 * them; h is requantised with the power-of-two rule.  Same arguments, layouts
 * and errors.  A scale that is not such a power of two is read as its FP32
 * exponent only (the result is then wrong; it is not checked). */
moe_status grouped_gemm_fp8_up_e8m0(const uint8_t* aq, const float* as, int a_rows,
                                    const int32_t* row_src, const int32_t* offsets,
                                    int n_groups, int total_rows, int d, int f,
                                    const uint8_t* w13, const float* w13_s,
                                    uint8_t* h, float* hs, void* stream);
moe_status grouped_gemm_fp8_down_e8m0(const uint8_t* h, const float* hs, const int32_t* offsets,
                                      int n_groups, int total_rows, int d, int f,
                                      const uint8_t* w2, const float* w2_s,
                                      uint16_t* y, void* stream);

/* ---- Backward of the layer (training) ----
 * The pages run all three GEMMs of each linear layer in FP8 (summary page
 * section 6: Fprop, Dgrad, Wgrad), cache the SwiGLU inputs in FP8 and
 * recompute SwiGLU in the backward, and regroup 1x128 tiles into 128x1 tiles
 * with power-of-two scales where a backward GEMM needs the other orientation
 * (book chapter 17; chapter 16 "Why transposition is not trivial").  Every
 * quantisation below uses the power-of-two rule of the E8M0 section above.
 *
 * Dgrad needs no entry point of its own: grouped_gemm_fp8_down computes
 * y = A * B^T for any (N, K) = (d, f) and, given the transposed weights
 * (moe_transpose_fp8_blocks), gives dH = dY * W2 (A = dY, B = W2^T [E+1, f, d])
 * and the expert-input gradient [dG, dU] * W13 (B = W13^T [E+1, d, 2f]).  The
 * token gradient is moe_combine with all weights 1.
 *
 * Wgrad operands are "K-major": a [C, Kp] byte matrix whose row c holds column
 * c of the operand for every row of every expert, expert e in the column range
 * [128 pb[e], 128 pb[e+1]), pb[e] = sum over earlier experts of
 * ceil(rows/128), padding columns zero codes; scales [Kp/128, C], one per
 * column and 128-row block; Kp = moe_wgrad_columns(total_rows, n_groups)
 * (columns past 128 pb[n_groups] are not written). */

/* grouped_gemm_fp8_up_train — grouped_gemm_fp8_up (same arguments, rules and
 * errors) that also writes the SwiGLU input the backward recomputes from
 * (book chapter 17 "SwiGLU recomputation"): [G, U] quantised in 1x128 tiles
 * with the forward's rule (amax/448):
 *   gu [total_rows, 2f] E4M3 out (columns [0, f) = G, [f, 2f) = U),
 *   gus [total_rows, 2f/128] FP32 out.
 * Always runs the tiled kernel. */
moe_status grouped_gemm_fp8_up_train(const uint8_t* aq, const float* as, int a_rows,
                                     const int32_t* row_src, const int32_t* offsets,
                                     int n_groups, int total_rows, int d, int f,
                                     const uint8_t* w13, const float* w13_s,
                                     uint8_t* h, float* hs, uint8_t* gu, float* gus, void* stream);

/* moe_transpose_fp8_blocks — for each of n_matrices [N, K] E4M3 matrices with
 * [N/128, K/128] block scales, the [K, N] transpose with [K/128, N/128] scales
 * (exact: a block scale serves both orientations).  Offline, once per weight
 * update.  w, wt device; wt must not alias w. */
moe_status moe_transpose_fp8_blocks(const uint8_t* w, const float* ws, int n_matrices, int N, int K,
                                    uint8_t* wt, float* wts, void* stream);

/* moe_combine_backward — gradients of moe_combine (book chapter 7 "Selecting
 * and combining experts"): for every token t and slot j,
 *   dy[pos[t][j]]     = BF16(w[t][j] * dout[t])      (FP32 product)
 *   dw[t][j]          = sum_c dout[t][c] * y[pos[t][j]][c]   (FP32 sum)
 *   dy[shared_row0+t] = dout[t]   (when shared_row0 >= 0)
 *   dout [T, d] BF16; y [rows, d] BF16 (the forward's expert outputs);
 *   pos, w [T, k]; dy [rows, d] BF16 out; dw [T, k] FP32 out.
 * rows = shared_row0 + T (T*k without a shared expert), as for moe_combine; a
 * slot whose pos lies outside [0, rows) (an unassigned slot) gets dw = 0 and
 * writes no dY row. */
moe_status moe_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                const float* w, int T, int k, int d, int32_t shared_row0,
                                uint16_t* dy, float* dw, void* stream);

/* moe_combine_backward_q — moe_combine_backward that also writes the 1x128
 * power-of-two FP8 copy of every dY row it writes (the Dgrad operand, book
 * chapter 17: dY enters the backward GEMMs in FP8), bit for bit what
 * fp8_quant_1x128_pow2 makes of dy, without reading dy back:
 *   dyq [rows, d] E4M3 codes, dys [rows, d/128] FP32 scales (rows written by
 *   this call only; other rows untouched).  Same arguments and errors
 *   otherwise. */
moe_status moe_combine_backward_q(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                  const float* w, int T, int k, int d, int32_t shared_row0,
                                  uint16_t* dy, float* dw, uint8_t* dyq, float* dys, void* stream);

/* moe_wgrad_columns — Kp of the K-major layout for total_rows rows in n_groups
 * groups: 128 * (total_rows / 128 + n_groups), an upper bound of
 * 128 pb[n_groups] that depends only on host-known sizes (0 on bad input). */
int moe_wgrad_columns(int total_rows, int n_groups);

/* moe_regroup_128x1 — the K-major 128x1 power-of-two FP8 copy (out [C, Kp],
 * out_s [Kp/128, C]) of one operand of Wgrad, from either
 *   xq, xs   a 1x128 FP8 tensor ([*, C] codes, [*, C/128] scales) whose row r
 *            of the grouped order is row row_src[r] (row r when NULL): the
 *            forward's cache of X, dequantised in FP32 and requantised; or
 *   x_bf16   a BF16 tensor [total_rows, C] in grouped order (dY)
 * (exactly one of xq and x_bf16).  offsets [n_groups + 1] as for the GEMMs.
 * MOE_ERR_UNSUPPORTED: n_groups > 1024, more than 65535 padded row blocks, or
 * C * Kp above 2^32 bytes. */
moe_status moe_regroup_128x1(const uint8_t* xq, const float* xs, const uint16_t* x_bf16,
                             const int32_t* row_src, const int32_t* offsets, int n_groups,
                             int total_rows, int C, uint8_t* out, float* out_s, void* stream);

/* moe_swiglu_backward — SwiGLU backward recomputed from the forward's FP8 cache
 * (book chapter 17 "SwiGLU recomputation").  Per row r of the grouped order
 * and column j < f, with g, u the cached [G, U] codes times their 1x128 scales
 * (FP32) and s = sigmoid(g), evaluated in FP64 and rounded once to FP32:
 *   h = g s u,  dG = dH u s (1 + g (1 - s)),  dU = dH g s
 *   gu, gus    [rows, 2f] E4M3 and [rows, 2f/128] FP32: the cache ([G, U])
 *   dh         [rows, f] BF16
 *   dgu, dgus  [rows, 2f] / [rows, 2f/128] out: [dG, dU], 1x128 power-of-two
 *              (the Dgrad operand)
 *   dgu_t, dgu_ts  K-major [2f, Kp] / [Kp/128, 2f] out: [dG, dU] in 128x1 tiles
 *   h_t, h_ts      K-major [f, Kp] / [Kp/128, f] out: h in 128x1 tiles
 * (the Wgrad operands of W13 and W2). */
moe_status moe_swiglu_backward(const uint8_t* gu, const float* gus, const uint16_t* dh,
                               const int32_t* offsets, int n_groups, int total_rows, int f,
                               uint8_t* dgu, float* dgus, uint8_t* dgu_t, float* dgu_ts,
                               uint8_t* h_t, float* h_ts, void* stream);

/* grouped_gemm_fp8_wgrad — weight gradients of all experts (summary page
 * section 6, Wgrad in FP8): for every group e with rows [offsets[e],
 * offsets[e+1]),
 *   dw[e][m][n] = sum over the group's rows r of A(r, m) * B(r, n)
 * where A and B are K-major 128x1 operands (moe_regroup_128x1,
 * moe_swiglu_backward): a_t [M, Kp] / a_ts [Kp/128, M], b_t [N, Kp] /
 * b_ts [Kp/128, N], Kp = moe_wgrad_columns(total_rows, n_groups), all scales
 * powers of two (they go to the block-scaled MFMA as E8M0 codes).
 *   dw [n_groups, M, N] FP32 out (zeros for a group without rows).
 * dW2 = grouped_gemm_fp8_wgrad(dY_t, H_t) with (M, N) = (d, f); dW13 =
 * grouped_gemm_fp8_wgrad([dG, dU]_t, X_t) with (M, N) = (2f, d). */
moe_status grouped_gemm_fp8_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t,
                                  const float* b_ts, const int32_t* offsets, int n_groups,
                                  int total_rows, int M, int N, float* dw, void* stream);

/* Measurement utilities (not steps of the layer): the roofs the layer's
 * kernels are bound by, measured on the device, to read a kernel's rate
 * against beside the datasheet peaks (5.0 PFLOP/s dense FP8, 8 TB/s).
 *
 * moe_roof_fp8_mfma — `workgroups` workgroups of 4 waves; every wave issues
 *   iters * 8 FP8 MFMAs (v_mfma_scale_f32_16x16x128_f8f6f4, 65536 FLOP each)
 *   back to back on 8 independent accumulators, operands in registers, no
 *   memory traffic: workgroups * 4 * iters * 8 * 65536 FLOP per call.
 *   sink [workgroups * 256] FP32 out (each thread's accumulator sum).
 * moe_roof_hbm_read — reads every byte of buf [bytes] (16-byte aligned,
 *   bytes % 16 == 0) once with 16-byte loads from `workgroups` workgroups of
 *   256 threads; sink [workgroups * 256] uint32 out (an XOR of the words each
 *   thread read).  Use a buffer much larger than the 256 MB last-level cache.
 * moe_roof_dma_read — the expert GEMMs' weight-load pattern alone: buf
 *   [rows, K] bytes (16-byte aligned, K a multiple of 128; the first
 *   32 * floor(bytes / (32 K)) rows are read).  `workgroups` workgroups of 8
 *   waves; each wave streams 32 rows K block by K block with direct
 *   global->LDS loads of whole 128-byte lines into an LDS ring, `ahead`
 *   (1, 2 or 4) blocks of 4 KB in flight per wave.  sink [workgroups * 512]
 *   uint32 out (K blocks each thread's wave streamed).
 * moe_roof_hbm_latency — one lane follows `steps` links of the chain in
 *   next [n] uint32 (caller-built: next[i] is the index of the entry read
 *   after entry i; an index >= n is clamped to n - 1) from entry `start`;
 *   time / steps is the latency of a dependent load.  sink [1] uint32 out
 *   (the last index).  Lay the chain over a buffer much larger than the
 *   last-level cache, one entry per 128-byte line, in random order.
 * All four: asynchronous on `stream`; the caller times them (HIP events).
 * Errors: MOE_ERR_INVALID_ARG for sizes or pointers outside the ranges above. */
moe_status moe_roof_fp8_mfma(int workgroups, int iters, float* sink, void* stream);
moe_status moe_roof_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                             void* stream);
moe_status moe_roof_dma_read(const void* buf, size_t bytes, int K, int ahead, int workgroups, uint32_t* sink,
                             void* stream);
moe_status moe_roof_hbm_latency(const uint32_t* next, size_t n, uint32_t start, int steps, uint32_t* sink,
                                void* stream);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
