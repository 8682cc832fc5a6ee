// Combine: each token's routed expert outputs weighted by its gates, plus the
// shared expert's output, in BF16 (the book's chapter 7 "Selecting and
// combining experts": the routed weights sum to one and the shared expert is
// added separately; chapter 15 "What combine must do": token identity is kept;
// chapter 17 "FP8 dispatch, BF16 combine").
//
// One workgroup per token; each thread owns 8 consecutive columns (16-byte
// loads of every source row, one 16-byte store).  The sum is FP32 in slot
// order, then the shared row, then the optional residual row (chapter 15
// lists the residual path among what combine adds), so the result is
// deterministic.  HBM-bound: (k + 1) BF16 rows read and one written per token.
// With k known at compile time all of a chunk's row loads are issued before
// the first is used.  The expert rows are read with non-temporal loads (each
// is read once; 0.468 -> 0.411 ms at T = 16384).
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ void add_row(float (&acc)[8], const uint4 v, float wj) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu)), acc[2 * i]);
    acc[2 * i + 1] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(u[i] >> 16)), acc[2 * i + 1]);
  }
}
__device__ __forceinline__ void add_row(float (&acc)[8], const uint4 v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
    acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
  }
}

// 16-byte load that does not allocate in the caches: each routed and shared
// row is read exactly once
typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const uint16_t* p) {
  const u32x4c v = __builtin_nontemporal_load(reinterpret_cast<const u32x4c*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// KC > 0: k == KC, unrolled; KC == 0: any k.
template <int KC>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int k, int d,
                                                      int rows, int shared_row0,
                                                      const uint16_t* __restrict__ residual,
                                                      uint16_t* __restrict__ out) {
  __shared__ int s_pos[16];
  __shared__ float s_w[16];
  const int t = blockIdx.x;
  const int kk = KC > 0 ? KC : k;
  const int tid = threadIdx.x;
  if (tid < kk) {
    const int p = pos[(size_t)t * kk + tid];
    const bool ok = p >= 0 && p < rows;   // an unassigned slot contributes nothing
    s_pos[tid] = ok ? p : 0;
    s_w[tid] = ok ? w[(size_t)t * kk + tid] : 0.0f;
  }
  __syncthreads();
  const int n8 = d / 8;
  for (int c = tid; c < n8; c += (int)blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if (KC > 0) {
      uint4 v[KC > 0 ? KC : 1];
#pragma unroll
      for (int j = 0; j < KC; ++j) v[j] = load_once(y + (size_t)s_pos[j] * d + c * 8);
      uint4 vs = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
      if (shared_row0 >= 0) vs = load_once(y + (size_t)(shared_row0 + t) * d + c * 8);
      if (residual) vr = *reinterpret_cast<const uint4*>(residual + (size_t)t * d + c * 8);
#pragma unroll
      for (int j = 0; j < KC; ++j) add_row(acc, v[j], s_w[j]);
      if (shared_row0 >= 0) add_row(acc, vs);
      if (residual) add_row(acc, vr);
    } else {
      for (int j = 0; j < k; ++j) add_row(acc, load_once(y + (size_t)s_pos[j] * d + c * 8), s_w[j]);
      if (shared_row0 >= 0) add_row(acc, load_once(y + (size_t)(shared_row0 + t) * d + c * 8));
      if (residual) add_row(acc, *reinterpret_cast<const uint4*>(residual + (size_t)t * d + c * 8));
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * d + c * 8) = o;
  }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int k,
                          int d, int shared_row0, const uint16_t* residual, uint16_t* out,
                          hipStream_t stream) {
  const int rows = T * k + (shared_row0 >= 0 ? T : 0);
  const int rlim = shared_row0 >= 0 ? shared_row0 + T : rows;
  // threads: the 8-column chunks of a row in equal shares of 128..256 when
  // there are such shares (224 x 4 for d = 7168), else 256
  const int n8 = d / 8;
  int nt = 256;
  for (int q = (n8 + 255) / 256; n8 / q >= 128; ++q)
    if (n8 % q == 0) { nt = n8 / q; break; }
  if (k == 8)
    hipLaunchKernelGGL(combine_kernel<8>, dim3(T), dim3(nt), 0, stream, y, pos, w, k, d, rlim, shared_row0,
                       residual, out);
  else
    hipLaunchKernelGGL(combine_kernel<0>, dim3(T), dim3(nt), 0, stream, y, pos, w, k, d, rlim, shared_row0,
                       residual, out);
  return hipGetLastError();
}

}  // namespace moe
