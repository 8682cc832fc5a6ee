// Grouping of (token, expert) assignments by expert, the single-GPU form of
// dispatch (the book's chapter 7 "Batches change what is active": assignments
// are grouped by expert so each expert runs one batched product; chapter 15
// "What dispatch must do": the rows keep the identity of their source token).
//
// A stable counting sort in three deterministic passes over blocks of 256
// tokens, with no order-dependent atomics:
//   count    per-block expert histogram (LDS counters; the totals do not depend
//            on the order of the increments)
//   scan     per-expert exclusive scan over blocks, then over experts -> offsets
//   scatter  rank of a token among the block's earlier tokens with the same
//            expert from an LDS bitmap (popcounts), row = offset + block base +
//            rank; row_token and pos written, shared rows are the identity
// and an optional gather that copies each token's FP8 row and scales to its
// k + 1 rows (the dispatch proper; the grouped GEMM can instead read the
// token rows through row_token).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PB = 256;  // tokens per block

size_t permute_workspace_bytes(int T, int E) {
  const size_t nb = (size_t)(T + PB - 1) / PB;
  return nb * (size_t)E * sizeof(int32_t);
}

__global__ __launch_bounds__(PB) void permute_count_kernel(const int32_t* __restrict__ idx, int T,
                                                           int k, int E,
                                                           int32_t* __restrict__ block_counts) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  const int t = blockIdx.x * PB + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) block_counts[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

// Single workgroup: thread e turns column e of the block counts into exclusive
// block bases (in place) and its total; then an exclusive scan over experts.
__global__ __launch_bounds__(256) void permute_scan_kernel(int32_t* __restrict__ block_counts,
                                                           int nb, int E, int T, int k,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int tot[256];
  __shared__ int wave_tot[4];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      const int c = block_counts[(size_t)b * E + e];
      block_counts[(size_t)b * E + e] = run;
      run += c;
    }
  }
  tot[e] = (e < E) ? run : 0;
  // exclusive scan of tot[0..255]: inclusive scan within each wave, then wave carries
  const int lane = e & 63, wave = e >> 6;
  int v = tot[e];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int carry = 0;
  for (int w = 0; w < wave; ++w) carry += wave_tot[w];
  const int excl = carry + v - tot[e];
  if (e < E) offsets[e] = excl;
  if (e == 0) {
    offsets[E] = T * k;
    offsets[E + 1] = T * k + T;
  }
}

__global__ __launch_bounds__(PB) void permute_scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                             int k, int E,
                                                             const int32_t* __restrict__ block_base,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ pos,
                                                             int32_t* __restrict__ row_token) {
  __shared__ uint32_t bits[256][PB / 32];
  __shared__ int base[256];
  const int tid = threadIdx.x;
  for (int i = tid; i < 256 * (PB / 32); i += PB) (&bits[0][0])[i] = 0u;
  if (tid < E) base[tid] = offsets[tid] + block_base[(size_t)blockIdx.x * E + tid];
  __syncthreads();
  const int t = blockIdx.x * PB + tid;
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&bits[e][word], bit);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      int p = -1;
      if (e >= 0 && e < E) {
        int rank = __popc(bits[e][word] & (bit - 1u));
        for (int w = 0; w < word; ++w) rank += __popc(bits[e][w]);
        p = base[e] + rank;
        row_token[p] = t;
      }
      pos[(size_t)t * k + j] = p;
    }
    row_token[(size_t)T * k + t] = t;
  }
}

// One destination row per workgroup: 16-byte chunks of the FP8 row, then the
// row's FP32 scales.
__global__ __launch_bounds__(256) void permute_gather_kernel(const int32_t* __restrict__ row_token,
                                                             const uint8_t* __restrict__ xq,
                                                             const float* __restrict__ xs, int T,
                                                             int d, uint8_t* __restrict__ xq_perm,
                                                             float* __restrict__ xs_perm) {
  const size_t r = blockIdx.x;
  // Rows left unassigned by out-of-range expert ids hold no token: clamp the
  // source so every read stays inside xq.
  const int src = min(max(row_token[r], 0), T - 1);
  const int n16 = d / 16;
  const uint4* s = reinterpret_cast<const uint4*>(xq + (size_t)src * d);
  uint4* o = reinterpret_cast<uint4*>(xq_perm + r * d);
  for (int c = threadIdx.x; c < n16; c += 256) o[c] = s[c];
  const int ns = d / 128;
  for (int c = threadIdx.x; c < ns; c += 256) xs_perm[r * ns + c] = xs[(size_t)src * ns + c];
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, const uint8_t* xq,
                          const float* xs, int d, int32_t* offsets, int32_t* pos,
                          int32_t* row_token, uint8_t* xq_perm, float* xs_perm, void* ws,
                          hipStream_t stream) {
  const int nb = (T + PB - 1) / PB;
  int32_t* block_counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(permute_count_kernel, dim3(nb), dim3(PB), 0, stream, idx, T, k, E,
                     block_counts);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, stream, block_counts, nb, E, T, k,
                     offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(PB), 0, stream, idx, T, k, E,
                     block_counts, offsets, pos, row_token);
  if (xq_perm != nullptr) {
    const size_t rows = (size_t)T * k + T;
    hipLaunchKernelGGL(permute_gather_kernel, dim3((unsigned)rows), dim3(256), 0, stream, row_token,
                       xq, xs, T, d, xq_perm, xs_perm);
  }
  return hipGetLastError();
}

// ---- allocation-free variant ----
// The per-block histograms of moe_permute_noalloc live in a file-scope device
// array of kPermuteScratchBytes, one copy per GPU for the life of the process.
// Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and that pointer is what
// the kernels receive.  The count kernel overwrites every entry a call uses,
// so nothing is cleared between calls; calls that overlap on one GPU share
// the array and race.
static __device__ __align__(256) int32_t scratch[kPermuteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU
}  // namespace

static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_permute_noalloc(const int32_t* idx, int T, int k, int E, const uint8_t* xq,
                                  const float* xs, int d, int32_t* offsets, int32_t* pos,
                                  int32_t* row_token, uint8_t* xq_perm, float* xs_perm,
                                  hipStream_t stream) {
  if (permute_workspace_bytes(T, E) > kPermuteScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_permute(idx, T, k, E, xq, xs, d, offsets, pos, row_token, xq_perm, xs_perm, ws, stream);
}

}  // namespace moe
