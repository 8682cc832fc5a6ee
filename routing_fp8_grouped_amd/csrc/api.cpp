// C ABI of libmoe: host-side validation, then launches on the caller's stream.
// Validation is synchronous and touches no device memory; an invalid call
// returns an error code before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local char g_err[512];

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, ...)                                 \
  do {                                                     \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

// Byte and BF16 matrices are accessed with 16-byte vector loads/stores; FP32
// and int32 arrays element by element.
#define REQUIRE_PTR_A(p, a)                                                   \
  do {                                                                        \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);   \
    if (!aligned((p), (a)))                                                   \
      return fail(MOE_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, (int)(a)); \
  } while (0)
#define REQUIRE_PTR(p) REQUIRE_PTR_A(p, 16)
#define REQUIRE_PTR4(p) REQUIRE_PTR_A(p, 4)

#define REQUIRE_ALIGNED4_OR_NULL(p)                                           \
  do {                                                                        \
    if ((p) != nullptr && !aligned((p), 4))                                   \
      return fail(MOE_ERR_INVALID_ARG, "%s is not 4-byte aligned", #p);       \
  } while (0)

moe_status check_route_params(const moe_route_params& p) {
  REQUIRE(p.n_experts >= 1 && p.n_experts <= 256, "n_experts=%d must be in [1, 256]", p.n_experts);
  REQUIRE(p.n_groups >= 1 && p.n_groups <= 64, "n_groups=%d must be in [1, 64]", p.n_groups);
  REQUIRE(p.n_experts % p.n_groups == 0, "n_experts=%d is not a multiple of n_groups=%d",
          p.n_experts, p.n_groups);
  REQUIRE(p.topk_groups >= 1 && p.topk_groups <= p.n_groups, "topk_groups=%d must be in [1, %d]",
          p.topk_groups, p.n_groups);
  REQUIRE(p.topk >= 1, "topk=%d must be >= 1", p.topk);
  REQUIRE(p.topk % p.topk_groups == 0, "topk=%d is not a multiple of topk_groups=%d", p.topk,
          p.topk_groups);
  const int per = p.n_experts / p.n_groups;
  REQUIRE(p.topk / p.topk_groups <= per, "topk/topk_groups=%d exceeds the %d experts of a group",
          p.topk / p.topk_groups, per);
  REQUIRE(p.topk <= p.topk_groups * per, "topk=%d exceeds the %d experts of the kept groups",
          p.topk, p.topk_groups * per);
  REQUIRE(std::isfinite(p.route_scale), "route_scale is not finite");
  if (p.topk > 16) return fail(MOE_ERR_UNSUPPORTED, "topk=%d > 16 is not implemented", p.topk);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_route(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d,
                     moe_route_params p, int32_t* idx, float* w, void* stream) {
  clear_error();
  REQUIRE(T >= 0, "T=%d is negative", T);
  moe_status s = check_route_params(p);
  if (s != MOE_OK) return s;
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / p.topk, "T*k overflows int32");
  REQUIRE((uint64_t)T * (uint64_t)d * 2u <= 0xFFFFFFFFull, "x of T=%d rows x d=%d exceeds 4 GiB", T, d);
  REQUIRE_PTR(x);
  REQUIRE_PTR(wg);
  REQUIRE_ALIGNED4_OR_NULL(bias);
  REQUIRE_PTR4(idx);
  REQUIRE_PTR4(w);
  return hip_status(moe::launch_route(x, wg, bias, T, d, p.n_experts, p.n_groups, p.topk_groups,
                                      p.topk, p.route_scale, idx, w,
                                      static_cast<hipStream_t>(stream)),
                    "moe_route launch");
}

size_t moe_route_workspace_bytes(int T, int E) {
  if (E < 1 || E > 256) return 0;
  return moe::route_workspace_bytes(T, E);
}

moe_status moe_route_ws(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d,
                        moe_route_params p, int32_t* idx, float* w, void* workspace,
                        size_t workspace_bytes, void* stream) {
  clear_error();
  REQUIRE(T >= 0, "T=%d is negative", T);
  moe_status s = check_route_params(p);
  if (s != MOE_OK) return s;
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / p.topk, "T*k overflows int32");
  REQUIRE((uint64_t)T * (uint64_t)d * 2u <= 0xFFFFFFFFull, "x of T=%d rows x d=%d exceeds 4 GiB", T, d);
  REQUIRE_PTR(x);
  REQUIRE_PTR(wg);
  REQUIRE_ALIGNED4_OR_NULL(bias);
  REQUIRE_PTR4(idx);
  REQUIRE_PTR4(w);
  const size_t need = moe::route_workspace_bytes(T, p.n_experts);
  if (need > 0) {
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0 || workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace %p of %zu bytes: %zu bytes, 4-byte aligned, needed", workspace,
                  workspace_bytes, need);
  }
  return hip_status(moe::launch_route_ws(x, wg, bias, T, d, p.n_experts, p.n_groups, p.topk_groups,
                                         p.topk, p.route_scale, idx, w,
                                         need > 0 ? static_cast<float*>(workspace) : nullptr,
                                         static_cast<hipStream_t>(stream)),
                    "moe_route_ws launch");
}

namespace {

moe_status quant_1x128_impl(const uint16_t* x, int rows, int cols, uint8_t* q, float* scale, bool pow2,
                            void* stream) {
  REQUIRE(rows >= 0, "rows=%d is negative", rows);
  REQUIRE(cols >= 128 && cols % 128 == 0, "cols=%d must be a positive multiple of 128", cols);
  if (rows == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(q);
  REQUIRE_PTR4(scale);
  return hip_status(moe::launch_quant_1x128(x, rows, cols, q, scale, pow2,
                                            static_cast<hipStream_t>(stream)),
                    pow2 ? "fp8_quant_1x128_pow2 launch" : "fp8_quant_1x128 launch");
}

moe_status quant_128x128_impl(const uint16_t* w, int N, int K, uint8_t* q, float* scale, bool pow2,
                              void* stream) {
  REQUIRE(N >= 0 && N % 128 == 0, "N=%d must be a non-negative multiple of 128", N);
  REQUIRE(K >= 128 && K % 128 == 0, "K=%d must be a positive multiple of 128", K);
  if (N == 0) return MOE_OK;
  if (N / 128 > 65535) return fail(MOE_ERR_UNSUPPORTED, "N/128=%d exceeds 65535", N / 128);
  REQUIRE_PTR(w);
  REQUIRE_PTR(q);
  REQUIRE_PTR4(scale);
  return hip_status(moe::launch_quant_128x128(w, N, K, q, scale, pow2,
                                              static_cast<hipStream_t>(stream)),
                    pow2 ? "fp8_quant_128x128_pow2 launch" : "fp8_quant_128x128 launch");
}

}  // namespace

moe_status fp8_quant_1x128(const uint16_t* x, int rows, int cols, uint8_t* q, float* scale,
                           void* stream) {
  clear_error();
  return quant_1x128_impl(x, rows, cols, q, scale, false, stream);
}

moe_status fp8_quant_1x128_pow2(const uint16_t* x, int rows, int cols, uint8_t* q, float* scale,
                                void* stream) {
  clear_error();
  return quant_1x128_impl(x, rows, cols, q, scale, true, stream);
}

moe_status fp8_quant_128x128(const uint16_t* w, int N, int K, uint8_t* q, float* scale,
                             void* stream) {
  clear_error();
  return quant_128x128_impl(w, N, K, q, scale, false, stream);
}

moe_status fp8_quant_128x128_pow2(const uint16_t* w, int N, int K, uint8_t* q, float* scale,
                                  void* stream) {
  clear_error();
  return quant_128x128_impl(w, N, K, q, scale, true, stream);
}

size_t moe_permute_workspace_bytes(int T, int k, int E) {
  (void)k;
  if (T <= 0 || E <= 0) return 0;
  return moe::permute_workspace_bytes(T, E);
}

}  // extern "C"

namespace {

// Arguments of moe_permute other than the workspace; MOE_OK with T = 0 means
// nothing is to be done (the caller returns before launching).
moe_status check_permute(const int32_t* idx, int T, int k, int E, const uint8_t* xq, const float* xs,
                         int d, int32_t* offsets, int32_t* pos, int32_t* row_token, uint8_t* xq_perm,
                         float* xs_perm) {
  REQUIRE(T >= 0, "T=%d is negative", T);
  REQUIRE(E >= 1 && E <= 256, "E=%d must be in [1, 256]", E);
  REQUIRE(k >= 1 && k <= 16 && k <= E, "k=%d must be in [1, min(16, E)]", k);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / (k + 1), "T*(k+1) overflows int32");
  REQUIRE_PTR4(idx);
  REQUIRE_PTR4(offsets);
  REQUIRE_PTR4(pos);
  REQUIRE_PTR4(row_token);
  if (xq_perm != nullptr) {
    REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
    REQUIRE_PTR(xq);
    REQUIRE_PTR4(xs);
    REQUIRE_PTR(xq_perm);
    REQUIRE_PTR4(xs_perm);
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_permute(const int32_t* idx, int T, int k, int E, const uint8_t* xq, const float* xs,
                       int d, int32_t* offsets, int32_t* pos, int32_t* row_token, uint8_t* xq_perm,
                       float* xs_perm, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  moe_status st = check_permute(idx, T, k, E, xq, xs, d, offsets, pos, row_token, xq_perm, xs_perm);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = moe::permute_workspace_bytes(T, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  REQUIRE(aligned(workspace, 4), "workspace is not 4-byte aligned");
  return hip_status(moe::launch_permute(idx, T, k, E, xq, xs, d, offsets, pos, row_token, xq_perm,
                                        xs_perm, workspace, static_cast<hipStream_t>(stream)),
                    "moe_permute launch");
}

moe_status moe_permute_noalloc(const int32_t* idx, int T, int k, int E, const uint8_t* xq,
                               const float* xs, int d, int32_t* offsets, int32_t* pos,
                               int32_t* row_token, uint8_t* xq_perm, float* xs_perm, void* stream) {
  clear_error();
  moe_status st = check_permute(idx, T, k, E, xq, xs, d, offsets, pos, row_token, xq_perm, xs_perm);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = moe::permute_workspace_bytes(T, E);
  if (need > moe::kPermuteScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "T=%d, E=%d need %zu bytes of scratch; moe_permute_noalloc holds %zu "
                "(ceil(T/256) * E <= %zu); use moe_permute with a workspace",
                T, E, need, moe::kPermuteScratchBytes, moe::kPermuteScratchBytes / sizeof(int32_t));
  return hip_status(moe::launch_permute_noalloc(idx, T, k, E, xq, xs, d, offsets, pos, row_token,
                                                xq_perm, xs_perm, static_cast<hipStream_t>(stream)),
                    "moe_permute_noalloc");
}

namespace {

moe_status check_gemm_shape(int n_groups, int total_rows, int d, int f) {
  REQUIRE(n_groups >= 1, "n_groups=%d must be >= 1", n_groups);
  if (n_groups > 1024) return fail(MOE_ERR_UNSUPPORTED, "n_groups=%d > 1024", n_groups);
  REQUIRE(total_rows >= 0, "total_rows=%d is negative", total_rows);
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  REQUIRE(f >= 128 && f % 128 == 0, "f=%d must be a positive multiple of 128", f);
  // the kernels address one expert's weights and the activation rows with
  // 32-bit byte offsets
  if ((uint64_t)2 * f * d > 0xFFFFFFFFull)
    return fail(MOE_ERR_UNSUPPORTED, "2f*d=%llu bytes per expert exceeds 4 GiB",
                (unsigned long long)2 * f * d);
  if ((uint64_t)total_rows * (uint64_t)(d > f ? d : f) > 0xFFFFFFFFull)
    return fail(MOE_ERR_UNSUPPORTED, "total_rows*max(d,f) exceeds 4 GiB");
  // tile list of the GEMM kernels: (m-tiles of 256 rows) x (n-tiles of 256
  // weight rows), indexed with 32-bit integers scaled by 8
  const uint64_t tiles = ((uint64_t)total_rows / 256 + (uint64_t)n_groups) *
                         (uint64_t)((d > f ? d : f) / 128);
  if (tiles >= (1ull << 28)) return fail(MOE_ERR_UNSUPPORTED, "too many GEMM tiles");
  return MOE_OK;
}

moe_status check_up(int d, const uint8_t* aq, const float* as, int a_rows, const int32_t* row_src,
                    const int32_t* offsets, int total_rows, const uint8_t* w13, const float* w13_s,
                    uint8_t* h, float* hs) {
  REQUIRE(a_rows >= 1, "a_rows=%d must be >= 1", a_rows);
  if ((uint64_t)a_rows * (uint64_t)d > 0xFFFFFFFFull)
    return fail(MOE_ERR_UNSUPPORTED, "a_rows*d exceeds 4 GiB");
  REQUIRE(row_src != nullptr || a_rows >= total_rows,
          "a_rows=%d < total_rows=%d without row_src", a_rows, total_rows);
  REQUIRE_PTR(aq);
  REQUIRE_PTR4(as);
  REQUIRE_ALIGNED4_OR_NULL(row_src);
  REQUIRE_PTR4(offsets);
  REQUIRE_PTR(w13);
  REQUIRE_PTR4(w13_s);
  REQUIRE_PTR(h);
  REQUIRE_PTR4(hs);
  return MOE_OK;
}

moe_status check_down(const uint8_t* h, const float* hs, const int32_t* offsets, const uint8_t* w2,
                      const float* w2_s, uint16_t* y) {
  REQUIRE_PTR(h);
  REQUIRE_PTR4(hs);
  REQUIRE_PTR4(offsets);
  REQUIRE_PTR(w2);
  REQUIRE_PTR4(w2_s);
  REQUIRE_PTR(y);
  return MOE_OK;
}

moe_status gemm_up_impl(const uint8_t* aq, const float* as, int a_rows, const int32_t* row_src,
                        const int32_t* offsets, int n_groups, int total_rows, int d, int f,
                        const uint8_t* w13, const float* w13_s, uint8_t* h, float* hs, bool e8m0,
                        void* stream) {
  moe_status s = check_gemm_shape(n_groups, total_rows, d, f);
  if (s != MOE_OK || total_rows == 0) return s;
  s = check_up(d, aq, as, a_rows, row_src, offsets, total_rows, w13, w13_s, h, hs);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_gemm_up(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d,
                                        f, w13, w13_s, h, hs, e8m0, static_cast<hipStream_t>(stream)),
                    e8m0 ? "grouped_gemm_fp8_up_e8m0 launch" : "grouped_gemm_fp8_up launch");
}

moe_status gemm_down_impl(const uint8_t* h, const float* hs, const int32_t* offsets, int n_groups,
                          int total_rows, int d, int f, const uint8_t* w2, const float* w2_s,
                          uint16_t* y, bool e8m0, void* stream) {
  moe_status s = check_gemm_shape(n_groups, total_rows, d, f);
  if (s != MOE_OK || total_rows == 0) return s;
  s = check_down(h, hs, offsets, w2, w2_s, y);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_gemm_down(h, hs, offsets, n_groups, total_rows, d, f, w2, w2_s, y,
                                          e8m0, static_cast<hipStream_t>(stream)),
                    e8m0 ? "grouped_gemm_fp8_down_e8m0 launch" : "grouped_gemm_fp8_down launch");
}

}  // namespace

moe_status grouped_gemm_fp8_up(const uint8_t* aq, const float* as, int a_rows,
                               const int32_t* row_src, const int32_t* offsets, int n_groups,
                               int total_rows, int d, int f, const uint8_t* w13,
                               const float* w13_s, uint8_t* h, float* hs, void* stream) {
  clear_error();
  return gemm_up_impl(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d, f, w13, w13_s, h,
                      hs, false, stream);
}

moe_status grouped_gemm_fp8_up_e8m0(const uint8_t* aq, const float* as, int a_rows,
                                    const int32_t* row_src, const int32_t* offsets, int n_groups,
                                    int total_rows, int d, int f, const uint8_t* w13,
                                    const float* w13_s, uint8_t* h, float* hs, void* stream) {
  clear_error();
  return gemm_up_impl(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d, f, w13, w13_s, h,
                      hs, true, stream);
}

moe_status grouped_gemm_fp8_up_train(const uint8_t* aq, const float* as, int a_rows,
                                     const int32_t* row_src, const int32_t* offsets, int n_groups,
                                     int total_rows, int d, int f, const uint8_t* w13,
                                     const float* w13_s, uint8_t* h, float* hs, uint8_t* gu,
                                     float* gus, void* stream) {
  clear_error();
  moe_status s = check_gemm_shape(n_groups, total_rows, d, f);
  if (s != MOE_OK || total_rows == 0) return s;
  s = check_up(d, aq, as, a_rows, row_src, offsets, total_rows, w13, w13_s, h, hs);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(gu);
  REQUIRE_PTR4(gus);
  if ((uint64_t)total_rows * (uint64_t)(2 * f) > 0xFFFFFFFFull)
    return fail(MOE_ERR_UNSUPPORTED, "total_rows*2f exceeds 4 GiB");
  return hip_status(moe::launch_gemm_up(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d,
                                        f, w13, w13_s, h, hs, false, static_cast<hipStream_t>(stream),
                                        gu, gus),
                    "grouped_gemm_fp8_up_train launch");
}

moe_status grouped_gemm_fp8_down(const uint8_t* h, const float* hs, const int32_t* offsets,
                                 int n_groups, int total_rows, int d, int f, const uint8_t* w2,
                                 const float* w2_s, uint16_t* y, void* stream) {
  clear_error();
  return gemm_down_impl(h, hs, offsets, n_groups, total_rows, d, f, w2, w2_s, y, false, stream);
}

moe_status grouped_gemm_fp8_down_e8m0(const uint8_t* h, const float* hs, const int32_t* offsets,
                                      int n_groups, int total_rows, int d, int f, const uint8_t* w2,
                                      const float* w2_s, uint16_t* y, void* stream) {
  clear_error();
  return gemm_down_impl(h, hs, offsets, n_groups, total_rows, d, f, w2, w2_s, y, true, stream);
}

moe_status grouped_gemm_fp8_swiglu(const uint8_t* aq, const float* as, int a_rows,
                                   const int32_t* row_src, const int32_t* offsets, int n_groups,
                                   int total_rows, int d, int f, const uint8_t* w13,
                                   const float* w13_s, const uint8_t* w2, const float* w2_s,
                                   uint8_t* h, float* hs, uint16_t* y, void* stream) {
  clear_error();
  moe_status s = check_gemm_shape(n_groups, total_rows, d, f);
  if (s != MOE_OK || total_rows == 0) return s;
  s = check_up(d, aq, as, a_rows, row_src, offsets, total_rows, w13, w13_s, h, hs);
  if (s != MOE_OK) return s;
  s = check_down(h, hs, offsets, w2, w2_s, y);
  if (s != MOE_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  s = hip_status(moe::launch_gemm_up(aq, as, a_rows, row_src, offsets, n_groups, total_rows, d, f,
                                     w13, w13_s, h, hs, false, st),
                 "grouped_gemm_fp8_swiglu launch (up)");
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_gemm_down(h, hs, offsets, n_groups, total_rows, d, f, w2, w2_s, y,
                                          false, st),
                    "grouped_gemm_fp8_swiglu launch (down)");
}

// ---- backward ----

moe_status moe_transpose_fp8_blocks(const uint8_t* w, const float* ws, int n_matrices, int N, int K,
                                    uint8_t* wt, float* wts, void* stream) {
  clear_error();
  REQUIRE(n_matrices >= 0, "n_matrices=%d is negative", n_matrices);
  REQUIRE(N >= 128 && N % 128 == 0, "N=%d must be a positive multiple of 128", N);
  REQUIRE(K >= 128 && K % 128 == 0, "K=%d must be a positive multiple of 128", K);
  if (n_matrices == 0) return MOE_OK;
  if (n_matrices > 65535 || N / 128 > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "n_matrices=%d or N/128 exceeds 65535", n_matrices);
  REQUIRE_PTR(w);
  REQUIRE_PTR4(ws);
  REQUIRE_PTR(wt);
  REQUIRE_PTR4(wts);
  REQUIRE(w != wt, "in-place transposition is not supported");
  return hip_status(moe::launch_transpose_blocks(w, ws, n_matrices, N, K, wt, wts,
                                                 static_cast<hipStream_t>(stream)),
                    "moe_transpose_fp8_blocks launch");
}

moe_status moe_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                const float* w, int T, int k, int d, int32_t shared_row0,
                                uint16_t* dy, float* dw, void* stream) {
  clear_error();
  REQUIRE(T >= 0, "T=%d is negative", T);
  REQUIRE(k >= 1 && k <= 16, "k=%d must be in [1, 16]", k);
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  REQUIRE(shared_row0 >= -1, "shared_row0=%d must be >= -1", shared_row0);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / (k + 1), "T*(k+1) overflows int32");
  REQUIRE_PTR(dout);
  REQUIRE_PTR(y);
  REQUIRE_PTR4(pos);
  REQUIRE_PTR4(w);
  REQUIRE_PTR(dy);
  REQUIRE_PTR4(dw);
  return hip_status(moe::launch_combine_backward(dout, y, pos, w, T, k, d, shared_row0, dy, dw, nullptr,
                                                 nullptr, static_cast<hipStream_t>(stream)),
                    "moe_combine_backward launch");
}

moe_status moe_combine_backward_q(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                  const float* w, int T, int k, int d, int32_t shared_row0, uint16_t* dy,
                                  float* dw, uint8_t* dyq, float* dys, void* stream) {
  clear_error();
  REQUIRE(T >= 0, "T=%d is negative", T);
  REQUIRE(k >= 1 && k <= 16, "k=%d must be in [1, 16]", k);
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  REQUIRE(shared_row0 >= -1, "shared_row0=%d must be >= -1", shared_row0);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / (k + 1), "T*(k+1) overflows int32");
  REQUIRE_PTR(dout);
  REQUIRE_PTR(y);
  REQUIRE_PTR4(pos);
  REQUIRE_PTR4(w);
  REQUIRE_PTR(dy);
  REQUIRE_PTR4(dw);
  REQUIRE_PTR(dyq);
  REQUIRE_PTR4(dys);
  return hip_status(moe::launch_combine_backward(dout, y, pos, w, T, k, d, shared_row0, dy, dw, dyq, dys,
                                                 static_cast<hipStream_t>(stream)),
                    "moe_combine_backward_q launch");
}

int moe_wgrad_columns(int total_rows, int n_groups) {
  if (total_rows < 0 || n_groups < 1) return 0;
  const long long c = 128LL * moe::wgrad_blocks_bound(total_rows, n_groups);
  return c > INT32_MAX ? 0 : (int)c;
}

namespace {

moe_status check_wgrad_layout(const int32_t* offsets, int n_groups, int total_rows, int C) {
  REQUIRE(n_groups >= 1, "n_groups=%d must be >= 1", n_groups);
  if (n_groups > 1024) return fail(MOE_ERR_UNSUPPORTED, "n_groups=%d > 1024", n_groups);
  REQUIRE(total_rows >= 0, "total_rows=%d is negative", total_rows);
  REQUIRE(C >= 128 && C % 128 == 0, "columns=%d must be a positive multiple of 128", C);
  if (moe::wgrad_blocks_bound(total_rows, n_groups) > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "more than 65535 padded row blocks");
  if ((uint64_t)C * (uint64_t)moe_wgrad_columns(total_rows, n_groups) > 0xFFFFFFFFull)
    return fail(MOE_ERR_UNSUPPORTED, "the K-major operand exceeds 4 GiB");
  REQUIRE_PTR4(offsets);
  return MOE_OK;
}

}  // namespace

moe_status moe_regroup_128x1(const uint8_t* xq, const float* xs, const uint16_t* x_bf16,
                             const int32_t* row_src, const int32_t* offsets, int n_groups,
                             int total_rows, int C, uint8_t* out, float* out_s, void* stream) {
  clear_error();
  moe_status s = check_wgrad_layout(offsets, n_groups, total_rows, C);
  if (s != MOE_OK || total_rows == 0) return s;
  REQUIRE((xq != nullptr) != (x_bf16 != nullptr), "exactly one of xq and x_bf16 must be given");
  if (xq) {
    REQUIRE_PTR(xq);
    REQUIRE_PTR4(xs);
    REQUIRE_ALIGNED4_OR_NULL(row_src);
  } else {
    REQUIRE_PTR(x_bf16);
    REQUIRE(row_src == nullptr, "row_src applies to the FP8 source only");
  }
  REQUIRE_PTR(out);
  REQUIRE_PTR4(out_s);
  return hip_status(moe::launch_regroup_128x1(xq, xs, x_bf16, row_src, offsets, n_groups, total_rows, C,
                                              moe_wgrad_columns(total_rows, n_groups), out, out_s,
                                              static_cast<hipStream_t>(stream)),
                    "moe_regroup_128x1 launch");
}

moe_status moe_swiglu_backward(const uint8_t* gu, const float* gus, const uint16_t* dh,
                               const int32_t* offsets, int n_groups, int total_rows, int f,
                               uint8_t* dgu, float* dgus, uint8_t* dgu_t, float* dgu_ts,
                               uint8_t* h_t, float* h_ts, void* stream) {
  clear_error();
  moe_status s = check_wgrad_layout(offsets, n_groups, total_rows, 2 * f);
  if (s != MOE_OK || total_rows == 0) return s;
  REQUIRE(f >= 128 && f % 128 == 0, "f=%d must be a positive multiple of 128", f);
  REQUIRE_PTR(gu);
  REQUIRE_PTR4(gus);
  REQUIRE_PTR(dh);
  REQUIRE_PTR(dgu);
  REQUIRE_PTR4(dgus);
  REQUIRE_PTR(dgu_t);
  REQUIRE_PTR4(dgu_ts);
  REQUIRE_PTR(h_t);
  REQUIRE_PTR4(h_ts);
  return hip_status(moe::launch_swiglu_backward(gu, gus, dh, offsets, n_groups, total_rows, f,
                                                moe_wgrad_columns(total_rows, n_groups), dgu, dgus,
                                                dgu_t, dgu_ts, h_t, h_ts, static_cast<hipStream_t>(stream)),
                    "moe_swiglu_backward launch");
}

moe_status grouped_gemm_fp8_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t,
                                  const float* b_ts, const int32_t* offsets, int n_groups,
                                  int total_rows, int M, int N, float* dw, void* stream) {
  clear_error();
  moe_status s = check_wgrad_layout(offsets, n_groups, total_rows, M > N ? M : N);
  if (s != MOE_OK) return s;
  REQUIRE(M >= 128 && M % 128 == 0, "M=%d must be a positive multiple of 128", M);
  REQUIRE(N >= 128 && N % 128 == 0, "N=%d must be a positive multiple of 128", N);
  REQUIRE_PTR(a_t);
  REQUIRE_PTR4(a_ts);
  REQUIRE_PTR(b_t);
  REQUIRE_PTR4(b_ts);
  REQUIRE_PTR(dw);
  return hip_status(moe::launch_wgrad(a_t, a_ts, b_t, b_ts, offsets, n_groups, M, N,
                                      moe_wgrad_columns(total_rows, n_groups), dw,
                                      static_cast<hipStream_t>(stream)),
                    "grouped_gemm_fp8_wgrad launch");
}

moe_status moe_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int k, int d,
                       int32_t shared_row0, const uint16_t* residual, uint16_t* out, void* stream) {
  clear_error();
  REQUIRE(T >= 0, "T=%d is negative", T);
  REQUIRE(k >= 1 && k <= 16, "k=%d must be in [1, 16]", k);
  REQUIRE(d >= 128 && d % 128 == 0, "d=%d must be a positive multiple of 128", d);
  REQUIRE(shared_row0 >= -1, "shared_row0=%d must be >= -1", shared_row0);
  if (T == 0) return MOE_OK;
  REQUIRE(T <= INT32_MAX / (k + 1), "T*(k+1) overflows int32");
  REQUIRE_PTR(y);
  REQUIRE_PTR4(pos);
  REQUIRE_PTR4(w);
  REQUIRE_PTR(out);
  REQUIRE(residual == nullptr || (reinterpret_cast<uintptr_t>(residual) & 15u) == 0,
          "residual is not 16-byte aligned");
  return hip_status(moe::launch_combine(y, pos, w, T, k, d, shared_row0, residual, out,
                                        static_cast<hipStream_t>(stream)),
                    "moe_combine launch");
}

moe_status moe_bias_update(const int32_t* offsets, int n_experts, float gamma, float* bias,
                           void* stream) {
  clear_error();
  REQUIRE(n_experts >= 1, "n_experts=%d must be >= 1", n_experts);
  REQUIRE(std::isfinite(gamma), "gamma is not finite");
  REQUIRE_PTR4(offsets);
  REQUIRE_PTR4(bias);
  return hip_status(moe::launch_bias_update(offsets, n_experts, gamma, bias,
                                            static_cast<hipStream_t>(stream)),
                    "moe_bias_update launch");
}

moe_status moe_roof_fp8_mfma(int workgroups, int iters, float* sink, void* stream) {
  clear_error();
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), "workgroups=%d must be in [1, 2^20]", workgroups);
  REQUIRE(iters >= 1, "iters=%d must be >= 1", iters);
  REQUIRE_PTR4(sink);
  return hip_status(moe::launch_roof_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream)),
                    "moe_roof_fp8_mfma launch");
}

moe_status moe_roof_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                             void* stream) {
  clear_error();
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), "workgroups=%d must be in [1, 2^20]", workgroups);
  REQUIRE(bytes >= 16 && bytes % 16 == 0, "bytes=%zu must be a positive multiple of 16", bytes);
  REQUIRE_PTR(buf);
  REQUIRE_PTR4(sink);
  return hip_status(moe::launch_roof_read(buf, bytes, workgroups, sink, static_cast<hipStream_t>(stream)),
                    "moe_roof_hbm_read launch");
}

moe_status moe_roof_dma_read(const void* buf, size_t bytes, int K, int ahead, int workgroups, uint32_t* sink,
                             void* stream) {
  clear_error();
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), "workgroups=%d must be in [1, 2^20]", workgroups);
  REQUIRE(K >= 128 && K % 128 == 0 && K <= (1 << 20), "K=%d must be a multiple of 128 in [128, 2^20]", K);
  REQUIRE(ahead == 1 || ahead == 2 || ahead == 4, "ahead=%d must be 1, 2 or 4", ahead);
  REQUIRE(bytes / ((size_t)K * 32) >= 1, "bytes=%zu holds no 32 rows of K=%d bytes", bytes, K);
  REQUIRE(bytes / ((size_t)K * 32) < (size_t)(1u << 31) - 8, "bytes=%zu: too many 32-row slabs", bytes);
  REQUIRE_PTR(buf);
  REQUIRE_PTR4(sink);
  return hip_status(moe::launch_roof_dma(buf, bytes, K, ahead, workgroups, sink, static_cast<hipStream_t>(stream)),
                    "moe_roof_dma_read launch");
}

moe_status moe_roof_hbm_latency(const uint32_t* next, size_t n, uint32_t start, int steps, uint32_t* sink,
                                void* stream) {
  clear_error();
  REQUIRE(n >= 1 && n <= 0xFFFFFFFFull, "n=%zu must be in [1, 2^32 - 1]", n);
  REQUIRE(start < n, "start=%u must be < n=%zu", start, n);
  REQUIRE(steps >= 1, "steps=%d must be >= 1", steps);
  REQUIRE_PTR4(next);
  REQUIRE_PTR4(sink);
  return hip_status(moe::launch_roof_chase(next, n, start, steps, sink, static_cast<hipStream_t>(stream)),
                    "moe_roof_hbm_latency launch");
}

}  // extern "C"
