// FP8 E4M3 quantisation with online per-tile scales: 1x128 activation tiles and
// 128x128 weight blocks (the "DeepSeek-V3" summary page, section 6, ingredients
// (a) fine-grained quantization and (d) online scaling; the book's chapter 16,
// "V3's grouping" and "Online scales").  Both kernels are HBM-bound streams:
// read BF16 once, write E4M3 once plus one FP32 per tile.
#include "common.h"
#include "kernels.h"

namespace moe {

// One 1x128 tile per 16 lanes; each lane owns 8 consecutive elements (one
// 16-byte load, one 8-byte store).  The amax reduction stays inside the 16-lane
// group (xor shuffles with masks < 16).  POW2 selects the power-of-two scale
// rule (smallest power of two not below amax/448).
template <bool POW2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x,
                                                          long n_tiles,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
  const long tile = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool valid = tile < n_tiles;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid) raw = *reinterpret_cast<const uint4*>(x + tile * 128 + sub * 8);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float s = tile_scale<POW2>(amax);
  uint2 out;
  out.x = f32x4_to_e4m3(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
  out.y = f32x4_to_e4m3(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
  if (valid) {
    *reinterpret_cast<uint2*>(q + tile * 128 + sub * 8) = out;
    if (sub == 0) scale[tile] = s;
  }
}

// One 128x128 block per workgroup: thread t owns 64 elements of row t/2
// (columns (t%2)*64 .. +64).  Block amax through wave shuffles and LDS.
template <bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ w,
                                                            int K,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  __shared__ float wave_amax[4];
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const size_t base = (size_t)(nb * 128 + r) * K + (size_t)kb * 128 + half * 64;
  float v[64];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 raw = *reinterpret_cast<const uint4*>(w + base + c * 8);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[c * 8 + 2 * i] = bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
      v[c * 8 + 2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
  const float s = tile_scale<POW2>(amax);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 out;
    out.x = f32x4_to_e4m3(v[c * 16 + 0] / s, v[c * 16 + 1] / s, v[c * 16 + 2] / s, v[c * 16 + 3] / s);
    out.y = f32x4_to_e4m3(v[c * 16 + 4] / s, v[c * 16 + 5] / s, v[c * 16 + 6] / s, v[c * 16 + 7] / s);
    out.z = f32x4_to_e4m3(v[c * 16 + 8] / s, v[c * 16 + 9] / s, v[c * 16 + 10] / s, v[c * 16 + 11] / s);
    out.w = f32x4_to_e4m3(v[c * 16 + 12] / s, v[c * 16 + 13] / s, v[c * 16 + 14] / s, v[c * 16 + 15] / s);
    *reinterpret_cast<uint4*>(q + base + c * 16) = out;
  }
  if (threadIdx.x == 0) scale[(size_t)nb * (K / 128) + kb] = s;
}

hipError_t launch_quant_1x128(const uint16_t* x, long rows, int cols, uint8_t* q, float* scale,
                              bool pow2, hipStream_t stream) {
  const long n_tiles = rows * (long)(cols / 128);
  const long blocks = (n_tiles + 15) / 16;
  if (pow2)
    hipLaunchKernelGGL(quant_1x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       n_tiles, q, scale);
  else
    hipLaunchKernelGGL(quant_1x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       n_tiles, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const uint16_t* w, int N, int K, uint8_t* q, float* scale,
                                bool pow2, hipStream_t stream) {
  if (pow2)
    hipLaunchKernelGGL(quant_128x128_kernel<true>, dim3(K / 128, N / 128), dim3(256), 0, stream, w,
                       K, q, scale);
  else
    hipLaunchKernelGGL(quant_128x128_kernel<false>, dim3(K / 128, N / 128), dim3(256), 0, stream, w,
                       K, q, scale);
  return hipGetLastError();
}

}  // namespace moe
