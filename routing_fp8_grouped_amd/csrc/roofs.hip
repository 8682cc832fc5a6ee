// Measured roofs of the two resources the layer's kernels are bound by: the
// FP8 matrix units (the expert GEMMs at large batches) and HBM reads (the
// expert weights streamed at decode sizes).  The datasheet peaks (5.0 PFLOP/s
// dense FP8, 8 TB/s) assume the nominal clock and ideal traffic; these two
// kernels measure what the chip sustains for the simplest form of each work,
// so that a kernel's fraction can be read against both.
//
// roof_mfma_kernel: every wave issues v_mfma_scale_f32_16x16x128_f8f6f4 back to
//   back on eight independent accumulators (no memory traffic, operands in
//   registers); 256 threads per workgroup, one wave per SIMD.
// roof_read_kernel: each workgroup streams a contiguous share of a buffer much
//   larger than the last-level cache with 16-byte loads, eight in flight per
//   lane, folded into one word so that nothing is dead.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void roof_mfma_kernel(int iters, float* __restrict__ sink) {
  const int tid = threadIdx.x;
  // small E4M3 codes (exponent field 1..2: 2^-6 .. 2^-5 magnitudes) keep every
  // sum far from overflow
  const int c = 0x08080808 + ((tid & 7) << 8);
  const v8i a = {c, c, c, c, c, c, c, c};
  const v8i b = {c ^ 0x00010000, c, c, c, c, c, c, c};
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma_fp8_16x16x128(a, b, acc[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  sink[(size_t)blockIdx.x * blockDim.x + tid] = s;
}

// Workgroup w streams its own contiguous share of the buffer in steps of
// 32 KB: thread t reads 16 bytes at step offset u * 4 KB + 16 t for u < 8, so
// every wave instruction reads 1 KB contiguous and each lane keeps eight loads
// in flight.
__global__ __launch_bounds__(256) void roof_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  constexpr size_t STEP = (size_t)U * 256;              // 16-byte words per step
  const size_t steps = n16 / STEP;
  const size_t s0 = steps * blockIdx.x / gridDim.x, s1 = steps * (blockIdx.x + 1) / gridDim.x;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t x = 0;
  for (size_t st = s0; st < s1; ++st) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p + st * STEP + threadIdx.x);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(q + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the tail shorter than one step, by the last workgroup
  if (blockIdx.x == gridDim.x - 1)
    for (size_t i = steps * STEP + threadIdx.x; i < n16; i += 256) {
      const uint4 v = p[i];
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

hipError_t launch_roof_mfma(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(roof_mfma_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_roof_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                            hipStream_t stream) {
  hipLaunchKernelGGL(roof_read_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
