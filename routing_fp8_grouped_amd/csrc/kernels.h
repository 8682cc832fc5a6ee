// Launch functions of the gfx950 kernels (host side of each .hip file).  Every
// function enqueues on `stream` and returns hipGetLastError(); arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_quant_1x128(const uint16_t* x, long rows, int cols, uint8_t* q, float* scale,
                              bool pow2, hipStream_t stream);
hipError_t launch_quant_128x128(const uint16_t* w, int N, int K, uint8_t* q, float* scale,
                                bool pow2, hipStream_t stream);

hipError_t launch_route(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d,
                        int E, int G, int M, int k, float route_scale, int32_t* idx, float* w,
                        hipStream_t stream);
size_t route_workspace_bytes(int T, int E);
hipError_t launch_route_ws(const uint16_t* x, const uint16_t* wg, const float* bias, int T, int d, int E,
                           int G, int M, int k, float route_scale, int32_t* idx, float* w, float* logits,
                           hipStream_t stream);

size_t permute_workspace_bytes(int T, int E);
// Largest workspace the allocation-free permute holds in its static device
// array (per-block histograms: ceil(T/256) * E int32).
constexpr size_t kPermuteScratchBytes = size_t(1) << 20;
hipError_t launch_permute_noalloc(const int32_t* idx, int T, int k, int E, const uint8_t* xq,
                                  const float* xs, int d, int32_t* offsets, int32_t* pos,
                                  int32_t* row_token, uint8_t* xq_perm, float* xs_perm,
                                  hipStream_t stream);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, const uint8_t* xq,
                          const float* xs, int d, int32_t* offsets, int32_t* pos,
                          int32_t* row_token, uint8_t* xq_perm, float* xs_perm, void* ws,
                          hipStream_t stream);

hipError_t launch_gemm_up(const uint8_t* aq, const float* as, int a_rows, const int32_t* row_src,
                          const int32_t* offsets, int n_groups, int total_rows, int d, int f,
                          const uint8_t* w13, const float* w13_s, uint8_t* h, float* hs,
                          bool e8m0, hipStream_t stream, uint8_t* gu = nullptr, float* gus = nullptr);
hipError_t launch_gemm_down(const uint8_t* h, const float* hs, const int32_t* offsets, int n_groups,
                            int total_rows, int d, int f, const uint8_t* w2, const float* w2_s,
                            uint16_t* y, bool e8m0, hipStream_t stream);

// Variants of the two expert GEMMs for few rows per group (weight streaming;
// launch_gemm_up/down choose them when total_rows <= 16 * n_groups and K is at
// most kSmallMaxK, the activation rows they stage in LDS).
constexpr int kSmallMaxK = 7168;
hipError_t launch_gemm_up_small(const uint8_t* aq, const float* as, int a_rows,
                                const int32_t* row_src, const int32_t* offsets, int n_groups,
                                int total_rows, int d, int f, const uint8_t* w13,
                                const float* w13_s, uint8_t* h, float* hs, bool pow2,
                                hipStream_t stream);
hipError_t launch_gemm_down_small(const uint8_t* h, const float* hs, const int32_t* offsets,
                                  int n_groups, int total_rows, int d, int f, const uint8_t* w2,
                                  const float* w2_s, uint16_t* y, hipStream_t stream);

hipError_t launch_bias_update(const int32_t* offsets, int E, float gamma, float* bias,
                              hipStream_t stream);

// Backward around the expert GEMMs (backward.hip).
hipError_t launch_transpose_blocks(const uint8_t* w, const float* ws, int G, int N, int K, uint8_t* wt,
                                   float* wts, hipStream_t stream);
hipError_t launch_combine_backward(const uint16_t* dout, const uint16_t* y, const int32_t* pos,
                                   const float* w, int T, int k, int d, int shared_row0, uint16_t* dy,
                                   float* dw, uint8_t* dyq, float* dys, hipStream_t stream);
int wgrad_blocks_bound(int total_rows, int n_groups);
hipError_t launch_regroup_128x1(const uint8_t* xq, const float* xs, const uint16_t* xb,
                                const int32_t* row_src, const int32_t* offsets, int n_groups,
                                int total_rows, int C, int Kp, uint8_t* out, float* out_s,
                                hipStream_t stream);
hipError_t launch_swiglu_backward(const uint8_t* guq, const float* gus, const uint16_t* dh,
                                  const int32_t* offsets, int n_groups, int total_rows, int f, int Kp,
                                  uint8_t* dguq, float* dgus, uint8_t* dgut, float* dguts, uint8_t* ht,
                                  float* hts, hipStream_t stream);

hipError_t launch_wgrad(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                        const int32_t* offsets, int n_groups, int M, int N, int Kp, float* out,
                        hipStream_t stream);

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int k,
                          int d, int shared_row0, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream);

// Measured roofs (roofs.hip): FP8 MFMA issue rate and HBM read streaming.
hipError_t launch_roof_mfma(int workgroups, int iters, float* sink, hipStream_t stream);
hipError_t launch_roof_dma(const void* buf, size_t bytes, int K, int ahead, int workgroups, uint32_t* sink,
                           hipStream_t stream);
hipError_t launch_roof_chase(const uint32_t* next, size_t n, uint32_t start, int steps, uint32_t* sink,
                             hipStream_t stream);
hipError_t launch_roof_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                            hipStream_t stream);

}  // namespace moe
