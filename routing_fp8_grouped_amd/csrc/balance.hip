// Auxiliary-loss-free load balancing: the per-expert bias controller ("DeepSeek-V3:
// the recipe, and the interconnect that shaped it", section "Auxiliary-loss-free
// balancing"; the "DeepSeek-V3" summary page, section 2; the book's chapter 8
// "V3's routing-only bias").  After a step, an expert whose load is above the
// mean has its selection bias lowered by gamma, one below the mean raised by
// gamma.  The load of expert e is its row count in the grouped buffer
// (offsets[e+1] - offsets[e]); the comparison with the mean is made exactly in
// integers (load * E against the total), the update in FP32.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ offsets, int E,
                                                          float gamma, float* __restrict__ bias) {
  const long long total = offsets[E];
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x) {
    const long long diff = (long long)(offsets[e + 1] - offsets[e]) * E - total;
    const float s = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] - gamma * s;   // gamma * s is exact: one rounding
  }
}

hipError_t launch_bias_update(const int32_t* offsets, int E, float gamma, float* bias,
                              hipStream_t stream) {
  const int blocks = (E + 255) / 256;
  hipLaunchKernelGGL(bias_update_kernel, dim3(blocks), dim3(256), 0, stream, offsets, E, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
