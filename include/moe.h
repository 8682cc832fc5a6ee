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
 * lower expert index).  Selection and gates are evaluated in FP64. */
moe_status moe_route(const uint16_t* x, const uint16_t* wg, const float* bias,
                     int T, int d, moe_route_params p,
                     int32_t* idx, float* w, void* stream);

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

/* moe_combine — out[t] = BF16( sum_j w[t][j] * y[pos[t][j]] + y[shared_row0 + t] )
 * (book chapter 7 "Selecting and combining experts"; chapter 15 "What combine
 * must do"), summed in FP32 in slot order.
 *   y            [rows, d] BF16 expert outputs
 *   pos, w       [T, k] rows and gates of each token
 *   shared_row0  first shared-expert row (T*k), or -1 for none
 *   out          [T, d] BF16 */
moe_status moe_combine(const uint16_t* y, const int32_t* pos, const float* w,
                       int T, int k, int d, int32_t shared_row0,
                       uint16_t* out, void* stream);

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

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
