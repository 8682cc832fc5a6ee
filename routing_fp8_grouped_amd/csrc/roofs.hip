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
// roof_dma_kernel: the expert GEMMs' weight-load pattern alone: rows of K
//   bytes, each wave streaming 32 rows K block by K block with direct
//   global->LDS loads of whole 128-byte lines (8 rows per 1 KB load) into its
//   own LDS ring, AHEAD blocks (AHEAD x 4 KB per wave, x 8 waves per CU) in
//   flight.  Its rate at AHEAD = 1, 2, 4 tests how many lines a CU keeps in
//   flight: by Little's law the rate per CU times the load latency.
// roof_chase_kernel: one lane follows a chain of dependent loads (each index
//   read is the next address), so the time per step is the latency of one
//   load that misses the caches.
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

// s_waitcnt vmcnt(4 n) (n blocks of 4 loads left in flight), lgkmcnt and
// expcnt unconstrained
__device__ __forceinline__ void roof_wait_blocks(int n) {
  if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
  else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F74);
  else if (n == 2) __builtin_amdgcn_s_waitcnt(0x0F78);
  else __builtin_amdgcn_s_waitcnt(0x0F7C);
}

template <int AHEAD>
__global__ __launch_bounds__(512, 1) void roof_dma_kernel(const uint8_t* __restrict__ w, int nslab, int K,
                                                          uint32_t* __restrict__ sink) {
  static_assert(AHEAD >= 1 && AHEAD <= 4, "at most 3 blocks counted by roof_wait_blocks");
  __shared__ __attribute__((aligned(16))) unsigned char ring[8][AHEAD + 1][4096];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KB = K / 128;
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) off[i] = (uint32_t)((i * 8 + (lane >> 3)) * K + (lane & 7) * 16);
  uint32_t blocks = 0;
  for (int l = blockIdx.x; l < (nslab + 7) / 8; l += gridDim.x) {
    const int slab = l * 8 + wave;
    if (slab >= nslab) continue;   // wave-uniform
    const uint8_t* base = w + (size_t)slab * 32 * K;
    auto issue = [&](int kb) {
      const uint32_t st = lds_addr(&ring[wave][kb % (AHEAD + 1)][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(base + (size_t)kb * 128, off[i], st + i * 1024);
    };
#pragma unroll
    for (int j = 0; j < AHEAD; ++j)
      if (j < KB) issue(j);
    for (int kb = 0; kb < KB; ++kb) {
      roof_wait_blocks(min(AHEAD - 1, KB - 1 - kb));   // block kb has landed
      if (kb + AHEAD < KB) issue(kb + AHEAD);          // into the stage of block kb - 1
      ++blocks;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = blocks;
}

__global__ void roof_chase_kernel(const uint32_t* __restrict__ next, uint32_t n, uint32_t start, int steps,
                                  uint32_t* __restrict__ sink) {
  if (threadIdx.x != 0) return;
  uint32_t i = start;
  for (int s = 0; s < steps; ++s) i = min(next[i], n - 1);   // the clamp keeps a bad chain in bounds
  sink[0] = i;
}

hipError_t launch_roof_dma(const void* buf, size_t bytes, int K, int ahead, int workgroups, uint32_t* sink,
                           hipStream_t stream) {
  const int nslab = (int)(bytes / ((size_t)K * 32));
  const uint8_t* w = static_cast<const uint8_t*>(buf);
  switch (ahead) {
    case 1: hipLaunchKernelGGL(roof_dma_kernel<1>, dim3(workgroups), dim3(512), 0, stream, w, nslab, K, sink); break;
    case 2: hipLaunchKernelGGL(roof_dma_kernel<2>, dim3(workgroups), dim3(512), 0, stream, w, nslab, K, sink); break;
    default: hipLaunchKernelGGL(roof_dma_kernel<4>, dim3(workgroups), dim3(512), 0, stream, w, nslab, K, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_roof_chase(const uint32_t* next, size_t n, uint32_t start, int steps, uint32_t* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(roof_chase_kernel, dim3(1), dim3(64), 0, stream, next, (uint32_t)n, start, steps, sink);
  return hipGetLastError();
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
